// MLA tree-verify attention for MI355X (gfx950): C-ABI entry points and kernels.
//
// Method: speculative-decoding verify attention over a latent KV cache. Draft
// tree nodes are checked against the full KV cache ("The Milestone Commit",
// Input Knowledge); prefix slots come first in a sequence's slot list and the
// draft tokens' slots follow ("The Checkpoint Report", Mistakes and Incorrect
// Assumptions). Each node sees the whole prefix plus itself and its ancestors.
// Split-K over the KV sequence with an online softmax and a separate reduction
// of the partials ("The Milestone Commit", Thinking Process; "The Commit That
// Locked In 6x Decode", 2. NSPLIT=64), a vectorised bf16 KV gather through the
// slot table ("The Commit That Locked In 6x Decode", 3. Vectorized bf16 Loads),
// and capture safety: no allocation and no host synchronisation inside a call
// ("The Commit That Locked In 6x Decode", 1. Capture-Safe Design).
//
// gfx950 design (see the header of verify_attn_partial_kernel for the layout):
//  - one workgroup = 4 waves (one per SIMD) = 128 query rows (rows are (node,
//    head) pairs of one sequence, r = t*H + h) x one split of the sequence's
//    KV positions; one workgroup per CU;
//  - KV tiles of 32 rows (36 KB) are gathered straight into LDS with 16-byte
//    direct-to-LDS loads, one slot-table lookup per row, two tiles ahead;
//  - S^T = K Q^T and O^T += V^T P^T on MFMA 32x32x16 bf16, so every lane holds
//    whole query rows of both the scores and the accumulator (the softmax state
//    of a row never leaves its lane pair); V^T comes from the K-major LDS tile
//    with the LDS transpose read; O stays in AGPRs;
//  - fp32 online softmax in base 2, tree mask from per-node 64-bit ancestor
//    masks built on the device from the parent pointers;
//  - at most 32 query rows per sequence: a small-row kernel (64-key tiles
//    gathered through VGPRs; see its header) instead;
//  - a split's partial result is its V average (weighted V sum over running
//    sum) rounded to bf16, with the fp32 running maximum and sum; a
//    log-sum-exp combine kernel merges the splits and rounds to bf16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/verify_attn.h"

namespace {

constexpr int KV_DIM = 576;
constexpr int V_DIM = 512;
constexpr int MAX_TREE = 64;

// Partial kernel geometry.
constexpr int NWAVES = 4;                  // waves per workgroup (one per SIMD)
constexpr int ROWS_PER_WAVE = 32;          // query rows per wave (MFMA 32x32 N)
constexpr int ROWS_PER_TILE = NWAVES * ROWS_PER_WAVE;  // 128 query rows per workgroup
constexpr int NK = 32;                     // KV rows per LDS tile
constexpr int ROWS_PER_LOAD_WAVE = NK / NWAVES;  // 8 KV rows gathered per wave
constexpr int CHUNK_GROUPS = KV_DIM / 64;  // 9 groups of 64 bf16 (8 x 16 B) per KV row
constexpr int GROUP_BYTES = NK * 128;      // one group for all NK rows: 4 KB
constexpr int TILE_BYTES = CHUNK_GROUPS * GROUP_BYTES;  // 36 KB
constexpr int NBUF = 4;                    // LDS ring of KV tiles (144 KB)
constexpr int SLOT_RING = 4;               // LDS ring of slot-table entries (tiles)
constexpr int QK_STEPS = KV_DIM / 16;      // 36 MFMA k-steps of 16 features
constexpr int PV_BLOCKS = V_DIM / 32;      // 16 output blocks of 32 features
constexpr float LAZY_RESCALE_LOG2 = 8.0f;  // running max is raised only past +8 (base 2)
constexpr int QK_AHEAD = 4;                // K operand reads in flight ahead of their MFMA
constexpr int PV_AHEAD = 4;                // V^T operand reads in flight ahead
constexpr int SM_PIECES = 16;              // softmax pieces interleaved with the next QK
// partials per batch of loads in the combine kernel: bf16 whole rows, bf16
// half rows, fp32 (about 100-110 VGPRs each: four waves per SIMD)
constexpr int COMBINE_BATCH = 12;
constexpr int COMBINE_BATCH_HALF = 16;
constexpr int COMBINE_BATCH_F32 = 8;
constexpr int COMBINE_BATCH_SLICE = 16;  // loads per lane and batch, four splits per load
constexpr int COMBINE_SLICES = 8;        // workgroups per row in the sliced combine (64 features each)
constexpr int QSTAGE_PIECES = KV_DIM / 2 / 8;  // 36 16-byte pieces per row and half
constexpr int QSTAGE_BYTES = ROWS_PER_WAVE * QSTAGE_PIECES * 16;  // 18 KB per wave
constexpr int QSTAGE_LOADS = QSTAGE_BYTES / 1024;                 // 18 direct-to-LDS loads
static_assert(NWAVES * QSTAGE_BYTES <= (NBUF - 2) * TILE_BYTES, "query staging fits tiles 2 and 3");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

struct Plan {
  int M;               // H*T rows per sequence
  int nxcd;            // XCDs the workgroups are dealt over
  int rows_per_tile;   // query rows per partial workgroup
  int nk;              // keys per KV tile of the partial kernel
  int row_tiles;       // ceil(M / ROWS_PER_TILE)
  int chunk;           // keys per split (multiple of NK)
  int max_splits;      // bound on the total number of splits
  int partial_blocks;  // multiple of 8
  int combine_wpr;     // waves per output row in the combine kernel (1, 2, 4, 8 or 16)
  int combine_halves;  // workgroups per row group (2: one per half of the features)
  int combine_slices;  // 8: the sliced combine (a workgroup per row and 64 features), else 1
  int combine_blocks;
  size_t part_o_bytes;
  size_t ws_bytes;
};

struct PartialArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* slot_idx;
  const int32_t* seq_lens;
  const int32_t* tree_parent;
  uint16_t* part_o;  // bf16 [max_splits][M][512]: V sum / running sum, RNE
  float* part_ml;    // [max_splits][M][2] = (running max (base 2, scaled), running sum)
  int B, H, T, M;
  int row_tiles, chunk, max_splits, max_seq_len;
  int nxcd;  // XCDs of the device (workgroup ids are dealt to them round-robin)
  int rows_per_tile;  // query rows per workgroup
  int64_t total_kv, pool_slots;
  float qk_scale_log2;  // sm_scale * log2(e)
};

struct AppendArgs {
  const uint16_t* kv_new;
  const int32_t* slot_idx;
  const int32_t* seq_lens;
  uint16_t* kv_pool;
  int B, T, max_seq_len;
  int64_t total_kv, pool_slots;
};

struct CompactArgs {
  const uint16_t* kv_pool;
  const int32_t* slot_idx;
  uint16_t* kv_dst;
  int64_t total_kv, pool_slots;
};

struct CombineArgs {
  const void* part_o;  // partial V averages: bf16 (bf16 path) or fp32 (fp32-input path)
  const float* part_ml;
  const int32_t* seq_lens;
  uint16_t* out;      // bf16 output, or
  float* out_f32;     // fp32 output (fp32-input path)
  int B, T, M, chunk, max_splits, max_seq_len;
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int clamp_len(int n, int T, int max_len) {
  return n < T ? T : (n > max_len ? max_len : n);
}

// Where global split g lives: sequence b, its first global split g0, the
// sequence's offset into slot_idx and its (clamped) length. One wave computes
// this on its own with a 64-lane scan over seq_lens; every wave of a
// workgroup gets the same answer.
struct SplitLoc {
  int b, g0, n_splits, len;
  int64_t seg;
};

__device__ bool locate_split(const int32_t* __restrict__ seq_lens, int B, int T, int max_len,
                             int chunk, int g, bool by_seq, SplitLoc* loc) {
  const int lane = threadIdx.x & 63;
  int gacc = 0;
  int64_t segacc = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int len = 0, ns = 0;
    if (b < B) {
      len = clamp_len(seq_lens[b], T, max_len);
      ns = (len + chunk - 1) / chunk;
    }
    int ns_inc = ns;
    long long len_inc = len;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int a = __shfl_up(ns_inc, d);
      const long long c = __shfl_up(len_inc, d);
      if (lane >= d) {
        ns_inc += a;
        len_inc += c;
      }
    }
    const int ns_first = gacc + ns_inc - ns;
    // by_seq: g is a sequence index; else g is a global split index.
    const bool hit = (b < B) && (by_seq ? (b == g) : (g >= ns_first && g < ns_first + ns));
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      loc->b = __shfl(b, src);
      loc->g0 = __shfl(ns_first, src);
      loc->n_splits = __shfl(ns, src);
      loc->len = __shfl(len, src);
      loc->seg = segacc + __shfl(len_inc - len, src);
      return true;
    }
    gacc += __shfl(ns_inc, 63);
    segacc += __shfl(len_inc, 63);
  }
  return false;
}

// Total number of splits over all sequences (same clamping as locate_split),
// computed by one wave; every wave of a workgroup gets the same answer.
__device__ int count_splits(const int32_t* __restrict__ seq_lens, int B, int T, int max_len, int chunk) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int ns = 0;
    if (b < B) ns = (clamp_len(seq_lens[b], T, max_len) + chunk - 1) / chunk;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ns += __shfl_xor(ns, d);
    total += ns;
  }
  return total;
}

// Work item of a partial-kernel workgroup. Items are (split, row tile) pairs
// over the splits of all sequences; the hardware deals workgroup ids to the
// device's nxcd XCDs round-robin, and each XCD gets a contiguous, equal share
// of the items that exist for these sequence lengths (the row tiles of one
// split then share that XCD's L2 for their KV reads). For B <= 64 one load of
// seq_lens serves both the item count and the split's location; larger
// batches scan twice.
// seq_lens[0] through the scalar cache (a uniform value: one load per wave on
// the scalar path, which the first vector loads of every workgroup do not
// queue behind). The wait is part of the statement, so the value is in its
// register when the statement ends.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ int load_first_len(const int32_t* seq_lens) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(seq_lens) : "memory");
  return v;
}
#pragma clang diagnostic pop

__device__ bool locate_item(const int32_t* __restrict__ seq_lens, int B, int T, int max_len, int chunk,
                            int max_splits, int row_tiles, int nxcd, int* g_out, int* rt_out, SplitLoc* loc) {
  const int lane = threadIdx.x & 63;
  if (B > 64) {
    int n_items = count_splits(seq_lens, B, T, max_len, chunk);
    n_items = __builtin_amdgcn_readfirstlane(min(n_items, max_splits) * row_tiles);
    const int per_xcd = (n_items + nxcd - 1) / nxcd;
    const int k_on_xcd = blockIdx.x / nxcd;
    const int logical = (blockIdx.x - k_on_xcd * nxcd) * per_xcd + k_on_xcd;
    if (k_on_xcd >= per_xcd || logical >= n_items) return false;
    *g_out = logical / row_tiles;
    *rt_out = logical - *g_out * row_tiles;
    return locate_split(seq_lens, B, T, max_len, chunk, *g_out, false, loc);
  }
  if (B == 1) {  // one sequence: its length is one uniform (scalar) load, no scan
    const int len = clamp_len(load_first_len(seq_lens), T, max_len);
    const int ns = (len + chunk - 1) / chunk;
    const int n_items = min(ns, max_splits) * row_tiles;
    const int per_xcd = (n_items + nxcd - 1) / nxcd;
    const int k_on_xcd = blockIdx.x / nxcd;
    const int logical = (blockIdx.x - k_on_xcd * nxcd) * per_xcd + k_on_xcd;
    if (k_on_xcd >= per_xcd || logical >= n_items) return false;
    const int g = logical / row_tiles;
    loc->b = 0;
    loc->g0 = 0;
    loc->n_splits = ns;
    loc->len = len;
    loc->seg = 0;
    *g_out = g;
    *rt_out = logical - g * row_tiles;
    return true;
  }
  int len = 0, ns = 0;
  if (lane < B) {
    len = clamp_len(seq_lens[lane], T, max_len);
    ns = (len + chunk - 1) / chunk;
  }
  int ns_inc = ns;
  long long len_inc = len;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int x = __shfl_up(ns_inc, d);
    const long long y = __shfl_up(len_inc, d);
    if (lane >= d) {
      ns_inc += x;
      len_inc += y;
    }
  }
  const int n_items = __builtin_amdgcn_readfirstlane(min(__shfl(ns_inc, 63), max_splits) * row_tiles);
  const int per_xcd = (n_items + nxcd - 1) / nxcd;
  const int k_on_xcd = blockIdx.x / nxcd;
  const int logical = (blockIdx.x - k_on_xcd * nxcd) * per_xcd + k_on_xcd;
  if (k_on_xcd >= per_xcd || logical >= n_items) return false;
  const int g = logical / row_tiles;
  const int ns_first = ns_inc - ns;
  const unsigned long long mask = __ballot(lane < B && g >= ns_first && g < ns_first + ns);
  if (!mask) return false;
  const int src = __ffsll((long long)mask) - 1;
  loc->b = __shfl(lane, src);
  loc->g0 = __shfl(ns_first, src);
  loc->n_splits = __shfl(ns, src);
  loc->len = __shfl(len, src);
  loc->seg = __shfl(len_inc - len, src);
  *g_out = g;
  *rt_out = logical - g * row_tiles;
  return true;
}

// Work item of a partial-kernel workgroup when the batch holds one sequence:
// the (split, row tile) items of a sequence max_len keys long, dealt to the
// XCDs as in locate_item. No device read, so the workgroup can issue its first
// loads before the sequence's length arrives; it ends once the length shows
// its split empty (lengths below max_len).
__device__ __forceinline__ bool deal_single(int max_len, int chunk, int max_splits, int row_tiles,
                                            int nxcd, int* g_out, int* rt_out) {
  const int ns = (max_len + chunk - 1) / chunk;
  const int n_items = min(ns, max_splits) * row_tiles;
  const int per_xcd = (n_items + nxcd - 1) / nxcd;
  const int k_on_xcd = blockIdx.x / nxcd;
  const int logical = (blockIdx.x - k_on_xcd * nxcd) * per_xcd + k_on_xcd;
  if (k_on_xcd >= per_xcd || logical >= n_items) return false;
  *g_out = logical / row_tiles;
  *rt_out = logical - *g_out * row_tiles;
  return true;
}

// Swizzle of the 16-byte chunk position inside a 128-byte row segment:
// position = (c % 8) ^ swz(row), where swz swaps bits 1 and 2 of row % 8 and
// flips bit 0 for rows 16..31 of a tile. Both operand access patterns of the
// kernel then run without LDS bank conflicts (measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter and by read throughput):
//  - QK, ds_read_b128 (lane l: row l%32, one chunk per lane half): eight
//    consecutive rows must land on eight distinct positions, and rows r and
//    r + 16 on positions that differ in bit 0;
//  - PV, ds_read_b64_tr_b16 (32 lanes: 4 consecutive rows x 4 consecutive
//    positions from a multiple of 4): rows r and r + 2 must differ in bit 2.
__device__ __forceinline__ int swz(int row) {
  return ((row & 1) | (((row >> 2) & 1) << 1) | (((row >> 1) & 1) << 2)) ^ ((row >> 4) & 1);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8. A field at its maximum does not wait.
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (exp << 4) | (lgkm << 8);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 7, 15));
}

// Workgroup barrier for LDS hand-off. Unlike __syncthreads() it does not wait
// for this wave's outstanding global loads (the next tile's prefetch); each
// wave first waits for its own share of the current tile with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 7, 0));  // this wave's LDS ops done
  asm volatile("s_barrier" ::: "memory");
}

// 32-bit LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS char*)(p);
}

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *(const LDS_AS bf16x8*)(uintptr_t)addr;
}

// Transposing LDS read: within each 16-lane group, lane 4r+c addresses 4
// consecutive bf16 of row r (columns 4c..4c+3); lane j receives column j of
// the group's 4 rows.
__device__ __forceinline__ bf16x4 lds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uintptr_t)addr);
}

// 16-byte global -> LDS load: lane l's 16 bytes from `gptr` land at LDS byte
// address lds_base + 16 * l (lds_base wave-uniform). Completion is tracked
// by this wave's vmcnt. Issued as an asm statement so that the compiler does
// not add its own conservative waits for it before unrelated LDS reads; the
// kernel orders the hand-off itself (wait_vmcnt + lds_barrier).
// M0 is clobbered; nothing else in this file's kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_base)
      : "memory", "m0");
}
// 4-byte global -> LDS load: lane l's 4 bytes land at lds_base + 4 * l.
__device__ __forceinline__ void load_to_lds4(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(gptr), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// acc += A * B with MFMA 32x32x16 bf16 on an accumulator held in AGPRs. The
// output accumulators of the partial kernel (256 per lane) live in AGPRs for
// the whole kernel; an asm statement pins them there. The compiler does not
// model the hazards of an asm MFMA, so the required wait states are explicit:
// two before it (an operand may have just been written by a VALU instruction)
// and mfma_drain() before its accumulator is read by anything but another
// accumulating MFMA.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_valu_gap() { asm volatile("s_nop 4"); }
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }
// acc *= s in place on the AGPRs (bracket with mfma_drain / mfma_valu_gap).
__device__ __forceinline__ void acc_scale(f32x16& acc, float s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc[i]), "=&v"(tmp)
                 : "v"(s));
  }
}

// Value of lane l ^ 32 (gfx950 permlane swap; plain VALU, no LDS).
__device__ __forceinline__ float xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, ((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
}

// Value of lane l ^ 16 (gfx950 permlane swap of 16-lane rows; plain VALU).
__device__ __forceinline__ float xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, ((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}

// Two floats to a pair of bf16 (round to nearest even), `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The two bf16 values of a packed pair, widened (exactly) to float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ------------------------------------------------------------ partial kernel
//
// One workgroup = 4 waves (one per SIMD) = 128 query rows (32 per wave) of one
// sequence x one split of that sequence's KV positions; one workgroup per CU.
//
// LDS: a ring of 4 KV tiles of 32 rows (36 KB each). KV row k (0..31) of a
// tile, 16-byte chunk c (0..71) of that row lives at
//   (c / 8) * 4096 + k * 128 + ((c % 8) ^ swz(k)) * 16.
// (In the prologue, the buffers of tiles 2 and 3 first stage the query.)
// Every wave gathers 8 rows of each tile: wave w loads KV rows 8w..8w+7 with 9
// direct-to-LDS loads of 1 KB (one per chunk group), lane -> (row 8w + lane/8,
// chunk position lane%8), spread over its QK MFMAs. The slot-table entries of
// those rows travel global -> LDS as well (one 4-byte load per lane into a
// small ring) two tiles before the gather that uses them. Past the end of the
// split the loads repeat the split's last row, so each wave issues exactly 10
// loads per tile and waits with a constant count.
//
// Per wave, per tile (32 query rows r, 32 keys j), MFMA 32x32x16 bf16:
//   S^T[j, r] = K[j, :] . Q[r, :]      36 k-steps of 16 features; A = K from LDS,
//     B = Q^T in VGPRs; lane l then holds row r = l%32, keys
//     8(i/4) + 4(l/32) + i%4, i < 16
//   O^T[n, r] += V^T[n, j] P^T[j, r]   16 blocks of 32 features x 2 k-steps of
//     16 keys; B = P^T is the bf16 score fragment itself (no lane exchange),
//     A = V^T comes from the K-major tile with the LDS transpose read, in the
//     same key order. O^T (256 accumulators per lane) stays in AGPRs; lane l
//     holds row r = l%32, features 32cb + 8(i/4) + 4(l/32) + i%4.
// Each K or V^T operand read from LDS feeds 32 query rows.
//
// Software pipeline: iteration `it` runs the QK of tile it+1 (36 MFMAs) with
// the online softmax of tile it issued between its MFMAs, then the PV of tile
// it (32 MFMAs). A raised running max rescales O after PV(it-1), as the online
// softmax requires. LDS buffers: tile it (PV), tile it+1 (QK), tiles it+2 and
// it+3 in flight. One barrier per iteration publishes tile it+1 and, every
// wave being done with iteration it-1, frees tile it-1's buffer for the gather
// of tile it+3, whose nine loads ride on the first half of the QK MFMAs (one
// every two), so the last of them has the rest of QK and all of PV to land.
template <bool ONE_SEQ, bool IDLE_WAVES>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void verify_attn_partial_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * TILE_BYTES + SLOT_RING * NWAVES * 256];
  __shared__ unsigned long long anc_s[MAX_TREE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ONE_SEQ (a batch of one sequence): the item comes from deal_single, and
  // the sequence's length and the slot entry of the split's first key are
  // loaded beside the first slot-table and query loads; until the length is
  // in, the split's end is bounded by max_seq_len. Otherwise locate_item.
  int g, rt;
  SplitLoc loc;
  int len_first = 0, slot_first = 0;
  if constexpr (ONE_SEQ) {
    if (!deal_single(a.max_seq_len, a.chunk, a.max_splits, a.row_tiles, a.nxcd, &g, &rt)) return;
    loc.b = 0;
    loc.g0 = 0;
    loc.n_splits = 0;
    loc.len = a.max_seq_len;
    loc.seg = 0;
  } else {
    if (!locate_item(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, a.max_splits, a.row_tiles, a.nxcd, &g, &rt, &loc))
      return;
  }
  g = __builtin_amdgcn_readfirstlane(g);
  rt = __builtin_amdgcn_readfirstlane(rt);
  loc.b = __builtin_amdgcn_readfirstlane(loc.b);
  loc.g0 = __builtin_amdgcn_readfirstlane(loc.g0);
  loc.len = __builtin_amdgcn_readfirstlane(loc.len);
  loc.seg = ((int64_t)__builtin_amdgcn_readfirstlane((int)(loc.seg >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)loc.seg);
  const int split = g - loc.g0;
  const int k0 = split * a.chunk;
  int k1 = min(k0 + a.chunk, loc.len);
  int P = loc.len - a.T;
  if constexpr (ONE_SEQ) {
    // uniform addresses (the compiler loads both through the scalar cache);
    // the first use, after the first query loads are issued, waits for them
    len_first = a.seq_lens[0];
    slot_first = a.slot_idx[k0 < a.total_kv ? k0 : a.total_kv - 1];
  }

  // ---- KV gather addressing
  const int ld_row = wave * ROWS_PER_LOAD_WAVE + (lane >> 3);
  const int ld_elem = 8 * ((lane & 7) ^ swz(ld_row));
  const int64_t slot_hi = a.total_kv - 1;
  const int pool_hi = (int)(a.pool_slots - 1 < (int64_t)INT32_MAX ? a.pool_slots - 1 : (int64_t)INT32_MAX);
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t ring_base = smem_base + NBUF * TILE_BYTES + wave * 256;
  // Slot-table entry of row r of this wave's 8 rows in the tile at key kt
  // (keys past the split end repeat its last key).
  auto slot_ptr = [&](int kt, int r) {
    int key = kt + wave * ROWS_PER_LOAD_WAVE + r;
    key = key < k1 ? key : k1 - 1;
    int64_t si = loc.seg + key;
    si = si < slot_hi ? si : slot_hi;
    return a.slot_idx + si;
  };
  // Slot entries of tile t -> LDS ring entry t % SLOT_RING (lane l: row l%8).
  auto issue_slots = [&](int t) {
    load_to_lds4(slot_ptr(k0 + t * NK, lane & 7), ring_base + (t % SLOT_RING) * (NWAVES * 256));
  };
  auto ring_slot = [&](int t) {
    return *(const LDS_AS int*)(uintptr_t)(ring_base + (t % SLOT_RING) * (NWAVES * 256) + 4 * (lane >> 3));
  };
  auto gather_src = [&](int slot) {
    slot = slot < 0 ? 0 : (slot > pool_hi ? pool_hi : slot);
    return a.kv + (int64_t)slot * KV_DIM + ld_elem;
  };
  auto gather_dst = [&](int t) {
    return smem_base + (t % NBUF) * TILE_BYTES + wave * (ROWS_PER_LOAD_WAVE * 128);
  };

  // Prologue loads, oldest first: the tree's parent pointers (wave 0, into
  // the ancestor-mask array, lane l at byte 4 l; lanes past T repeat node
  // T-1) and the slot entries of tiles 0 and 1 (lane: row lane/8 of this
  // wave's 8); the first half of this wave's query block into LDS; once the
  // slot entries are in, the gathers of tiles 0 and 1; then the second half
  // of the query block.
  const uint32_t anc_base = lds_addr(anc_s);
  if (wave == 0) load_to_lds4(a.tree_parent + (int64_t)loc.b * a.T + min(lane, a.T - 1), anc_base);
  int s_pro[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) s_pro[t] = *slot_ptr(k0 + t * NK, lane >> 3);
  // Query fragments (B operand of S^T = K Q^T): lane l holds row l%32,
  // features 16 ks + 8 (l/32) .. +7 of k-step ks, i.e. 16-byte piece
  // 2 ks + l/32 of its row. A wave without query rows only gathers its share
  // of the KV (see the loop below).
  const int row0 = rt * ROWS_PER_TILE + wave * ROWS_PER_WAVE;
  const bool wave_active = row0 < a.M;  // wave-uniform
  const int qrow = row0 + (lane & 31);
  const bool row_ok = qrow < a.M;
  const int hl = lane >> 5;  // lane half
  bf16x8 qf[QK_STEPS];
  // The query block passes through LDS in two halves (pieces 0..35 and
  // 36..71 of each of the wave's 32 rows), in a region of the ring buffers of
  // tiles 2 and 3, which are free until the QK of tile 0. Read straight into
  // the MFMA layout, each load instruction would touch 32 rows; staged, each
  // direct-to-LDS load reads 1 KB of consecutive query bytes. Staging slot
  // s = 36 r + p' holds piece p' ^ qswz(r) of row r (a permutation inside
  // aligned groups of four pieces), so that the MFMA-layout reads of eight
  // consecutive rows fall on eight distinct 16-byte positions and rows r and
  // r + 16 on positions that differ in bit 0 (the rules of swz above).
  const uint32_t qstage = smem_base + 2 * TILE_BYTES + wave * QSTAGE_BYTES;
  auto qswz = [](int r) { return ((r >> 1) & 3) ^ ((r >> 4) & 1); };
  // A load whose first row is past M is replaced by zeros written to its
  // staging slots (the waits below count younger loads only, so they just
  // get looser). Rows past M in the other loads repeat row 0. Either way a
  // row past M only feeds its own scores, weights and output column, which
  // are never stored.
  auto q_stage = [&](int half) {
#pragma unroll
    for (int j = 0; j < QSTAGE_LOADS; ++j) {
      if (row0 + (j * 64) / QSTAGE_PIECES >= a.M) {  // wave-uniform
        *(LDS_AS u32x4*)(uintptr_t)(qstage + j * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        continue;
      }
      const int slot = j * 64 + lane;
      const int r = slot / QSTAGE_PIECES;
      const int p = (slot - r * QSTAGE_PIECES) ^ qswz(r);
      const int grow = row0 + r < a.M ? row0 + r : 0;  // rows past M read row 0
      load_to_lds16(a.q + ((int64_t)loc.b * a.M + grow) * KV_DIM + half * (KV_DIM / 2) + 8 * p,
                    qstage + j * 1024);
    }
  };
  auto q_read = [&](int half) {
    const int r = lane & 31;
#pragma unroll
    for (int k = 0; k < QK_STEPS / 2; ++k) {
      const int p = 2 * k + hl;
      qf[half * (QK_STEPS / 2) + k] = lds_read_b128(qstage + (r * QSTAGE_PIECES + (p ^ qswz(r))) * 16);
    }
  };
  // A wave without query rows skips the staging loads (the waits below only
  // get looser).
  if (wave_active) q_stage(0);

  if constexpr (ONE_SEQ) {
    // With the length in: a split past the sequence's end leaves (once its
    // loads have landed: the query staging writes LDS); rows of tiles 0 and 1
    // past the end take the split's first key's slot, so that only this
    // sequence's KV rows are read (they are masked like the repeated last row
    // of a short split).
    loc.len = clamp_len(len_first, a.T, a.max_seq_len);
    if (k0 >= loc.len) {
      wait_vmcnt<0>();
      return;
    }
    k1 = min(k0 + a.chunk, loc.len);
    P = loc.len - a.T;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (k0 + t * NK + wave * ROWS_PER_LOAD_WAVE + (lane >> 3) >= k1) s_pro[t] = slot_first;
  }

  // Steady-state load order (iteration i: slots of tile i+5, gather of tile
  // i+3) for i = -3, -2: the gathers of tiles 0 and 1. Forming their row
  // addresses waits for the slot entries (and the first query half).
  const uint16_t* src_pro[2] = {gather_src(s_pro[0]), gather_src(s_pro[1])};
  asm volatile("" ::"v"(src_pro[0]), "v"(src_pro[1]));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    issue_slots(t + 2);
    const uint16_t* src = src_pro[t];
    const uint32_t dst = gather_dst(t);
#pragma unroll
    for (int j = 0; j < CHUNK_GROUPS; ++j) load_to_lds16(src + 64 * j, dst + j * GROUP_BYTES);
  }
  wait_vmcnt<2 * (CHUNK_GROUPS + 1)>();  // first query half in LDS (the gathers may still fly)
  asm volatile("" ::: "memory");
  q_read(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 7, 0));  // read out before the second half lands
  asm volatile("" ::: "memory");
  if (wave_active) q_stage(1);

  // While the second half and tiles 0 and 1 land (work kept off the path
  // from their arrival to the first MFMA):
  // - Ancestor masks of this sequence's tree (bit u of anc[t]: node u is t or
  //   an ancestor of t), by pointer jumping over the lanes of wave 0: after
  //   round k a node's mask holds its ancestors within distance 2^(k+1) - 1,
  //   and up[t] is its ancestor at distance 2^(k+1) (or -1). Six rounds cover
  //   depth 63. Parent pointers outside [-1, t-1] make t a root. The parent
  //   pointers landed with the first query half (they are older loads); every
  //   lane reads its pointer before the masks overwrite the array.
  if (wave == 0) {
    const int parent = *(const LDS_AS int*)(uintptr_t)(anc_base + 4 * lane);
    int up = (parent >= 0 && parent < lane && lane < a.T) ? parent : -1;
    unsigned long long m = lane < a.T ? (1ull << lane) : 0ull;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int src = up >= 0 ? up : lane;
      const unsigned long long m_up = __shfl(m, src);
      const int up_up = __shfl(up, src);
      if (up >= 0) {
        m |= m_up;
        up = up_up;
      }
    }
    if (lane < a.T) anc_s[lane] = m;
  }
  // - O = 0 in its AGPRs (the empty asm statements make the zeros exist here).
  f32x16 o[PV_BLOCKS];
#pragma unroll
  for (int cb = 0; cb < PV_BLOCKS; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
    asm volatile("" : "+a"(o[cb]));
  }

  wait_vmcnt<0>();  // second query half, and with it tiles 0 and 1, landed
  asm volatile("" ::: "memory");
  q_read(1);

  // Operand read offsets inside a tile (the chunk group is added as a constant).
  //  QK k-step ks reads chunk 2 ks + l/32 of key row l%32: group ks/4,
  //  position 2 (ks%4) + l/32.
  int qk_off[4];
  {
    const int kr = lane & 31;
#pragma unroll
    for (int j = 0; j < 4; ++j) qk_off[j] = kr * 128 + (((2 * j + hl) ^ swz(kr)) << 4);
  }
  //  PV block cb, key half kh: per 16-lane group q = l/16, lane 4 r + c
  //  addresses features 32 cb + 16 (q%2) + 4c .. +3 of key row
  //  16 kh + 8 rd + 4 (q/2) + r (rd = 0, 1 for the two halves of the operand):
  //  chunk 4 cb + 2 (q%2) + c/2 -> group cb/2, position 4 (cb%2) + 2 (q%2) + c/2.
  int pv_off[2][2][2];  // [kh][cb % 2][rd]
  {
    const int q = lane >> 4, r = (lane & 15) >> 2, c = lane & 3;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const int row = 16 * kh + 8 * rd + 4 * (q >> 1) + r;
          const int pos = 4 * cp + 2 * (q & 1) + (c >> 1);
          pv_off[kh][cp][rd] = row * 128 + ((pos ^ swz(row)) << 4) + 8 * (c & 1);
        }
  }

  float m_run = -INFINITY;  // running reference max (base-2 scaled scores)
  float l_run = 0.f;        // this lane's share of the running sum


  const int ntiles = (k1 - k0 + NK - 1) / NK;
  // ---- online softmax (base 2) of one tile's scores `sv`, in pieces that run
  // between the MFMAs of the next tile's QK. Piece st < SM_PIECES.
  f32x16 sv;                  // scores of the tile, then its weights
  int sm_kt = 0;              // first key of the tile
  float mx = 0.f, alpha = 1.f;
  bool any_raise = false;
  bf16x8 pb0 = {}, pb1 = {};  // bf16 weights: the PV B operand for keys of i < 8 / i >= 8
  auto sm_piece = [&](int st) __attribute__((always_inline)) {
    if (st == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] *= a.qk_scale_log2;
    } else if (st == 1) {
      if (sm_kt + NK > k1 || sm_kt + NK > P) {  // the tile reaches the split end or the tree
        const unsigned long long anc = anc_s[row_ok ? qrow / a.H : 0];
        const int kb0 = sm_kt + 4 * hl;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb0 + 8 * (i >> 2) + (i & 3);
          const int u = key - P;
          // bitwise, branch-free: the selects stay in place
          const bool vis = (key < k1) & ((u < 0) | (((anc >> (u & 63)) & 1ull) != 0));
          sv[i] = vis ? sv[i] : -INFINITY;
        }
      }
    } else if (st == 2) {
      mx = fmaxf(fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]))),
                 fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])), fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
    } else if (st == 3) {
      mx = fmaxf(mx, xor32(mx));  // lanes l and l^32 hold the same query row
      const bool raise = mx > m_run + LAZY_RESCALE_LOG2;
      // O needs rescaling only in rows that already hold weights: a row whose
      // running max was -inf has O = 0 (its first finite max is the common case
      // at the first tile of a split).
      any_raise = __ballot(raise & (m_run != -INFINITY)) != 0;
      alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;  // m_run = -inf -> 0
      m_run = raise ? mx : m_run;
      l_run *= alpha;
    } else if (st < 12) {
      const float mu = (m_run == -INFINITY) ? 0.f : m_run;
      const int i = 2 * (st - 4);
      sv[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
      sv[i + 1] = __builtin_amdgcn_exp2f(sv[i + 1] - mu);
    } else if (st == 12) {
      pb0 = bf16x8{(__bf16)sv[0], (__bf16)sv[1], (__bf16)sv[2], (__bf16)sv[3],
                   (__bf16)sv[4], (__bf16)sv[5], (__bf16)sv[6], (__bf16)sv[7]};
    } else if (st == 13) {
      pb1 = bf16x8{(__bf16)sv[8], (__bf16)sv[9], (__bf16)sv[10], (__bf16)sv[11],
                   (__bf16)sv[12], (__bf16)sv[13], (__bf16)sv[14], (__bf16)sv[15]};
    } else if (st == 14 || st == 15) {
      // The running sum uses the same bf16-rounded weights that enter O.
      const u32x4 w = __builtin_bit_cast(u32x4, st == 14 ? pb0 : pb1);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += __builtin_bit_cast(float, w[i] << 16) + __builtin_bit_cast(float, w[i] & 0xffff0000u);
      l_run += acc;
    }
  };

  // ---- S^T = K Q^T for tile t: 36 MFMAs, with the nine gather loads of tile
  // t+2 (one every 2 MFMAs over the first half, so that the last of them has
  // the second half of QK and all of PV to land) and, when `with_softmax`,
  // the softmax pieces of the previous tile (one every 2 MFMAs) in between.
  auto qk_tile = [&](int t, bool with_softmax) __attribute__((always_inline)) {
    const uint32_t cur = smem_base + (t % NBUF) * TILE_BYTES;
    uint32_t qb[4];  // per-tile base addresses; the chunk group goes in the immediate offset
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = cur + qk_off[j];
    auto kread = [&](int ks) { return lds_read_b128(qb[ks & 3] + (ks >> 2) * GROUP_BYTES); };
    bf16x8 kbuf[QK_AHEAD];
#pragma unroll
    for (int ks = 0; ks < QK_AHEAD; ++ks) kbuf[ks] = kread(ks);
    __builtin_amdgcn_sched_barrier(0);  // the operand reads go out before the slot read
    const int slot_next = ring_slot(t + 2);
    const uint32_t gdst = gather_dst(t + 2);
    issue_slots(t + 4);
    const uint16_t* gsrc = a.kv;
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      const bf16x8 kv = kbuf[ks % QK_AHEAD];
      if (ks + QK_AHEAD < QK_STEPS) kbuf[ks % QK_AHEAD] = kread(ks + QK_AHEAD);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qf[ks], s, 0, 0, 0);
      if (ks == 2) gsrc = gather_src(slot_next);  // first needed at ks = 3
      if ((ks & 1) == 1 && ks >= 3 && ks < 3 + 2 * CHUNK_GROUPS)  // ks = 3, 5, .., 19
        load_to_lds16(gsrc + 64 * ((ks - 3) >> 1), gdst + ((ks - 3) >> 1) * GROUP_BYTES);
      if (with_softmax && (ks & 1) == 0 && (ks >> 1) < SM_PIECES) sm_piece(ks >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    return s;
  };

  // ---- O^T += V^T P^T for tile t: 32 MFMAs, key half 0 (B = pb0) over the
  // 16 feature blocks, then key half 1 (B = pb1).
  auto pv_tile = [&](int t) __attribute__((always_inline)) {
    const uint32_t cur = smem_base + (t % NBUF) * TILE_BYTES;
    uint32_t vb[2][2][2];  // per-tile base addresses (chunk group in the immediate offset)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) vb[kh][cp][rd] = cur + pv_off[kh][cp][rd];
    auto vread = [&](int st) {  // step st = 16 kh + cb
      const int cb = st & 15, kh = st >> 4;
      const bf16x4 v0 = lds_read_tr(vb[kh][cb & 1][0] + (cb >> 1) * GROUP_BYTES);
      const bf16x4 v1 = lds_read_tr(vb[kh][cb & 1][1] + (cb >> 1) * GROUP_BYTES);
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vbuf[PV_AHEAD];
#pragma unroll
    for (int st = 0; st < PV_AHEAD; ++st) vbuf[st] = vread(st);
    mfma_valu_gap();  // pb0 / pb1 were written by VALU instructions
#pragma unroll
    for (int st = 0; st < 2 * PV_BLOCKS; ++st) {
      const bf16x8 vt = vbuf[st % PV_AHEAD];
      if (st + PV_AHEAD < 2 * PV_BLOCKS) vbuf[st % PV_AHEAD] = vread(st + PV_AHEAD);
      mfma_acc(o[st & 15], vt, st < 16 ? pb0 : pb1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // IDLE_WAVES (some row tile holds at most 96 rows): a wave without query
  // rows runs no MFMA. It only gathers its share of every tile, with the same
  // loads, waits and barriers as the loop below, and leaves after the last
  // barrier. (Without idle waves the instance keeps the loop's code as it is.)
  if (IDLE_WAVES && !wave_active) {
    auto gather_only = [&](int t) {  // the loads qk_tile(t) issues
      const int slot_next = ring_slot(t + 2);
      const uint32_t gdst = gather_dst(t + 2);
      issue_slots(t + 4);
      const uint16_t* gsrc = gather_src(slot_next);
#pragma unroll
      for (int j = 0; j < CHUNK_GROUPS; ++j) load_to_lds16(gsrc + 64 * j, gdst + j * GROUP_BYTES);
    };
    lds_barrier();
    gather_only(0);
    for (int it = 0; it + 1 < ntiles; ++it) {
      wait_vmcnt<CHUNK_GROUPS + 1>();
      lds_barrier();
      gather_only(it + 1);
    }
    wait_vmcnt<0>();
    lds_barrier();  // the epilogue's barrier
    return;
  }

  // Tile 0: publish it (every load of this wave so far has landed; the
  // barrier also ends every wave's query reads from the staging region),
  // then its QK (carrying the gather of tile 2).
  lds_barrier();  // tile 0 complete; ancestor masks visible
  sv = qk_tile(0, false);
  // Iteration it: QK of tile it+1 with the softmax of tile it in between, then
  // PV of tile it. Own loads are issued in the order (iteration i) slots of
  // tile i+5, gather of tile i+3; at the top of iteration it the gather of
  // tile it+1 and, before it, the slots of tile it+3 have landed once at most
  // 10 younger loads are out. The barrier publishes tile it+1 and, every wave
  // being done with iteration it-1, frees tile it-1's buffer for the gather of
  // tile it+3.
  for (int it = 0; it < ntiles; ++it) {
    sm_kt = k0 + it * NK;
    f32x16 sn;
    if (it + 1 < ntiles) {
      wait_vmcnt<CHUNK_GROUPS + 1>();
      lds_barrier();
      sn = qk_tile(it + 1, true);
    } else {
#pragma unroll
      for (int st = 0; st < SM_PIECES; ++st) sm_piece(st);
    }
    if (any_raise) {  // O (PV up to tile it-1) *= alpha
      mfma_drain();
#pragma unroll
      for (int cb = 0; cb < PV_BLOCKS; ++cb) acc_scale(o[cb], alpha);
      mfma_valu_gap();
    }
    pv_tile(it);
    sv = sn;
  }
  wait_vmcnt<0>();  // no load outlives the workgroup, and no gather lands in LDS after this
  mfma_drain();     // O is read below
  lds_barrier();    // every wave is done with the tile buffers, which now stage the partial rows
  if (!IDLE_WAVES && !wave_active) return;
  // ---- partial results of this split: the V average (0 for a row with every
  // key of the split masked), rounded to bf16, and the running maximum and sum.
  // The lane holds 4 features of each 8-feature chunk of its row; the wave's
  // 32 rows pass through LDS (row r: 1 KB, chunk c at position c ^ r, which
  // spreads the writes of 32 rows and the reads of one row evenly over the
  // banks) and leave one row per store instruction, 1 KB contiguous.
  // The lane's row and half are formed anew here (an asm statement the
  // compiler neither hoists nor merges), so that nothing derived from the lane
  // index has to stay live across the loop.
  int el;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(el));
  const int er = el & 31, ehl = el >> 5;
  const bool erow_ok = row0 + er < a.M;
  float l_row;
  {  // l_run + xor32(l_run), with the lane half taken from el
    const unsigned u = __builtin_bit_cast(unsigned, l_run);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_row = l_run + __builtin_bit_cast(float, ehl ? sw[0] : sw[1]);
  }
  const float inv = (erow_ok && l_row > 0.f) ? 1.0f / l_row : 0.f;
  const uint32_t stage = smem_base + wave * (ROWS_PER_WAVE * V_DIM * 2);
#pragma unroll
  for (int cb = 0; cb < PV_BLOCKS; ++cb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int c = 4 * cb + i4;  // features 8c + 4 hl .. +3
      *(LDS_AS u32x2*)(uintptr_t)(stage + er * (V_DIM * 2) + ((c ^ er) << 4) + 8 * ehl) =
          u32x2{pack_bf16x2(o[cb][4 * i4] * inv, o[cb][4 * i4 + 1] * inv),
                pack_bf16x2(o[cb][4 * i4 + 2] * inv, o[cb][4 * i4 + 3] * inv)};
    }
  const int nrows = min(ROWS_PER_WAVE, a.M - row0);  // wave-uniform, >= 1
  uint16_t* po = a.part_o + ((int64_t)g * a.M + row0) * V_DIM + 8 * el;
  for (int r = 0; r < nrows; ++r) {
    const u32x4 v = *(const LDS_AS u32x4*)(uintptr_t)(stage + r * (V_DIM * 2) + ((el ^ r) << 4));
    *reinterpret_cast<u32x4*>(po + (int64_t)r * V_DIM) = v;
  }
  if (erow_ok && ehl == 0) {
    const int64_t rowid = (int64_t)g * a.M + row0 + er;
    a.part_ml[2 * rowid] = m_run;
    a.part_ml[2 * rowid + 1] = l_row;
  }
}

// ------------------------------------------------- fp32-input partial kernel
//
// The same split-K partial results as verify_attn_partial_kernel, for binary32
// q and KV rows (the data type of the first, fp32 kernel of "The Checkpoint
// Report", Architecture of the Report), computed in fp32 throughout on MFMA
// 16x16x4 f32: no operand is rounded to a narrower type, the softmax weights
// included. The output partials have the same layout, so the same combine
// merges them (with an fp32 output).
//
// One workgroup = 4 waves x 16 query rows (64 rows of one sequence) x one
// split; one workgroup per CU. LDS: a ring of 3 KV tiles of 16 rows (36 KB
// each: 2,304 bytes per row). Row r of a tile, 16-byte piece c (0..143) lives
// at r * 2304 + (c ^ (r % 16)) * 16 (the XOR stays inside aligned groups of
// 16 pieces). Wave w gathers rows 4w .. 4w+3 of each tile with nine
// direct-to-LDS loads of 1 KB (consecutive LDS bytes, so lane -> (row, piece)
// follows the layout).
//
// Per wave, per tile (16 query rows n, 16 keys m), MFMA 16x16x4 f32 with the
// reduction index k = lane group g = lane / 16:
//   S^T[m, n] += K[m, f] Q[n, f]    f = 16 c + 4 g + i, MFMA step (c, i):
//     lane (m = l%16, g) gives K[m, f] (one 16-byte LDS read per chunk c
//     serves 4 steps) and Q[n = l%16, f] (held in 144 VGPRs); lane l then
//     holds S for row l%16, keys 4 g + i.
//   O^T[e, n] += V[k, e] P[n, k]    k = 4 g + i, step i, 16-feature block e:
//     B = P is the lane's own weight for key 4 g + i (no exchange). Block e
//     holds the features 64 (e / 4) + 4 m + e % 4 (m = 0..15), so that one
//     16-byte LDS read of lane (m, g) - features 64 J + 4 m .. +3 of key row
//     4 g + i - gives the A operands of blocks 4 J .. 4 J + 3. O (128 fp32 per
//     lane) stays in AGPRs; lane (n, g) holds, in register j of block e, the
//     feature 64 (e / 4) + 16 g + 4 j + e % 4 of row n, so the four blocks of
//     a group store one contiguous 16-byte piece per register.
// The XOR layout keeps both read patterns free of bank conflicts: the 16-byte
// K reads of 8 consecutive rows land on 8 distinct positions of a 128-byte
// window, and the 16 lanes of a V read that share a key row read 16 distinct
// positions of one 256-byte window.
constexpr int F_NK = 16;                          // keys per tile
constexpr int F_ROWS_PER_WAVE = 16;               // query rows per wave (MFMA N)
constexpr int F_ROWS_PER_TILE = NWAVES * F_ROWS_PER_WAVE;  // 64
constexpr int F_ROW_BYTES = KV_DIM * 4;           // 2,304
constexpr int F_TILE_BYTES = F_NK * F_ROW_BYTES;  // 36 KB
constexpr int F_NBUF = 3;
constexpr int F_PIECES = KV_DIM / 4;              // 144 16-byte pieces per row
constexpr int F_CHUNKS = KV_DIM / 16;             // 36 QK chunks of 16 features
constexpr int F_LOADS = F_NK / NWAVES * F_ROW_BYTES / 1024;  // 9 gather loads per wave and tile
constexpr int F_PV_BLOCKS = V_DIM / 16;           // 32 blocks of 16 features
static_assert(F_PIECES % 16 == 0, "the piece XOR stays inside a row");
static_assert(F_LOADS * 1024 == F_NK / NWAVES * F_ROW_BYTES, "whole loads per band");

struct PartialF32Args {
  const float* q;
  const float* kv;
  const int32_t* slot_idx;
  const int32_t* seq_lens;
  const int32_t* tree_parent;
  float* part_o;   // [max_splits][M][512]: V sum / running sum
  float* part_ml;  // [max_splits][M][2] = (running max, running sum)
  int B, H, T, M;
  int row_tiles, chunk, max_splits, max_seq_len;
  int nxcd;
  int64_t total_kv, pool_slots;
  float qk_scale_log2;
};

// acc += a * b (MFMA 16x16x4 f32) on an AGPR accumulator. No wait states in
// front: in the fp32 kernel's PV loop A comes straight from an LDS read and B
// was written by VALU before a mfma_valu_gap(); build.py checks the generated
// code for a VALU write to a source of these MFMAs just before them.
__device__ __forceinline__ void mfma16_acc(f32x4& acc, float a, float b) {
  asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_scale4(f32x4& acc, float s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc[i]), "=&v"(tmp)
                 : "v"(s));
  }
}

// ------------------------------------------------- small-row partial kernel
//
// The same split-K partial results for calls with at most 32 query rows per
// sequence (H*T <= 32: one TP8 rank's 8 heads verifying up to 4 draft tokens,
// plain decode included; "The Commit That Locked In 6x Decode", 2. NSPLIT=64
// for TP8 Occupancy). There the 128-row workgroup above leaves most of its
// MFMA rows empty; here a workgroup takes the sequence's rows in one or two
// 16-row MFMA blocks and all four waves work on every row. (The kernel also
// runs with several row tiles of at most 32 rows sharing a split, but then
// every compute unit gathers each key row of the split again, and the gather,
// not the arithmetic, bounds these calls: measured slower than the 128-row
// kernel from 40 rows up.)
//  - QK: wave w computes the scores of keys 16w .. 16w+15 of a 64-key tile for
//    all rows, S^T = K Q^T on MFMA 16x16x32 bf16 (A = 16 key rows from LDS,
//    B = Q^T held in AGPRs for the whole split);
//  - the tile's row maxima are exchanged through LDS; every wave then applies
//    the same online-softmax update (base 2, running maximum raised only past
//    +8) to its own keys and writes their bf16 weights to a shared LDS block;
//  - PV: wave w accumulates output features 128w .. 128w+127 of every row over
//    all 64 keys, O^T += V^T P^T on the same MFMA, with V^T read from the
//    K-major tile by the LDS transpose read and P^T from the weight block.
//    O (up to 64 fp32 per lane) stays in VGPRs and the query block (up to 144
//    registers) in AGPRs, from which the QK MFMAs read it.
// LDS: two 64-key tiles (72 KB each): key row k, 16-byte chunk c at
//   (c / 8) * 8192 + k * 128 + ((c % 8) ^ sm_swz(k)) * 16,
// sm_swz(k) = (k % 4) + 4 (((k / 4) ^ (k / 8)) % 2), a bijection of bits 0-2
// of k when bit 3 is fixed and of bits 1 and 3 when bits 0 and 2 are fixed.
// A 16-byte LDS read serves eight consecutive lanes per cycle; the 8-byte
// transpose read serves the lanes of a half-wave with lane bit 2 clear, then
// those with it set. So the QK reads (eight consecutive key rows, one chunk)
// and the PV transpose reads (per cycle: key rows 8G + 4h + r and 8(G+1) +
// 4h + r, r in {0, 2} or {1, 3}, two chunks each) land on distinct banks, as
// do the weight block's writes and reads (the same swizzle by row).
// The gather goes through VGPRs: a global load into VGPRs and an LDS write
// move random rows at several times the rate of the direct-to-LDS load on
// gfx950 (measured per compute unit, from L2). Wave w loads key rows 16w ..
// 16w+15 of tile t+1 with 18 loads of 16 bytes per lane (72 VGPRs) right
// after the barrier that frees their buffer (the top of iteration t) and
// writes them into it after PV; the slot entries come a tile earlier.
constexpr int SM_NK = 64;                                  // keys per tile
constexpr int SM_ROWS = 32;                                // query rows per workgroup (at most)
constexpr int SM_GROUP_BYTES = SM_NK * 128;                // one chunk group of the 64 rows: 8 KB
constexpr int SM_TILE_BYTES = CHUNK_GROUPS * SM_GROUP_BYTES;  // 72 KB
constexpr int SM_QK_STEPS = KV_DIM / 32;                   // 18 k-steps of 32 features
constexpr int SM_FB = V_DIM / NWAVES / 16;                 // 8 output blocks of 16 features per wave
constexpr int SM_LOADS = 2 * CHUNK_GROUPS;                 // 18 gather loads per wave and tile
constexpr int SM_P_BYTES = SM_ROWS * SM_NK * 2;            // bf16 weights of a tile: [row][key]
constexpr int SM_MAX_M = SM_ROWS;  // H*T up to which the plan takes this kernel (one row tile)
constexpr int SM_LDS = 2 * SM_TILE_BYTES + SM_P_BYTES + NWAVES * SM_ROWS * 4;
static_assert(SM_LDS + MAX_TREE * 8 <= 160 * 1024, "small-row kernel LDS");

__device__ __forceinline__ int sm_swz(int k) { return (k & 3) | ((((k >> 2) ^ (k >> 3)) & 1) << 2); }

// acc += a * b, MFMA 16x16x32 bf16 with the B operand (the query fragment,
// loop-invariant) held in AGPRs and the accumulator in VGPRs: the query block
// stays out of the VGPRs, which hold O and the gather in flight. The compiler
// does not model an asm MFMA's latency: its accumulator is read by VALU
// instructions only after mfma_drain_acc(); A comes from an LDS read and B is
// never written in the loop.
__device__ __forceinline__ void mfma16_qk(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// The same with a zero accumulator (C is the inline constant 0, so no VALU
// instruction writes it just before).
__device__ __forceinline__ void mfma16_qk_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
}
// The wait states of mfma_drain(), taking the accumulators of the asm MFMAs
// above as operands: a plain drain orders nothing for the compiler, which
// would be free to move the first VALU reads of these values above it.
template <int N>
__device__ __forceinline__ void mfma_drain_acc(f32x4 (&acc)[N][2]) {
  if constexpr (N == 1)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0][0]), "+v"(acc[0][1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));
}

__device__ __forceinline__ void lds_write_b128(uint32_t addr, const u32x4& v) { *(LDS_AS u32x4*)(uintptr_t)addr = v; }

// NRB: 16-row MFMA blocks of query rows per workgroup (1: up to 16 rows, 2: up to 32).
template <int NRB>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void verify_attn_partial_small_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[SM_LDS];
  __shared__ unsigned long long anc_s[MAX_TREE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int g, rt;
  SplitLoc loc;
  if (!locate_item(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, a.max_splits, a.row_tiles, a.nxcd, &g, &rt, &loc)) return;
  g = __builtin_amdgcn_readfirstlane(g);
  rt = __builtin_amdgcn_readfirstlane(rt);
  loc.b = __builtin_amdgcn_readfirstlane(loc.b);
  loc.g0 = __builtin_amdgcn_readfirstlane(loc.g0);
  loc.len = __builtin_amdgcn_readfirstlane(loc.len);
  loc.seg = ((int64_t)__builtin_amdgcn_readfirstlane((int)(loc.seg >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)loc.seg);
  const int k0 = (g - loc.g0) * a.chunk;
  const int k1 = min(k0 + a.chunk, loc.len);
  const int P = loc.len - a.T;
  const int ntiles = (k1 - k0 + SM_NK - 1) / SM_NK;

  const uint32_t smem_base = lds_addr(smem);
  const uint32_t p_base = smem_base + 2 * SM_TILE_BYTES;  // bf16 weights [32 rows][64 keys]
  const uint32_t rmax_base = p_base + SM_P_BYTES;         // fp32 [32 rows][4 waves]
  const int64_t slot_hi = a.total_kv - 1;
  const int pool_hi = (int)(a.pool_slots - 1 < (int64_t)INT32_MAX ? a.pool_slots - 1 : (int64_t)INT32_MAX);

  // Rows of this workgroup: local row lr = 16 rb + (lane % 16) is query row
  // rt * rows_per_tile + lr of the sequence (rows past the tile or M are zero).
  const int rpt = a.rows_per_tile;
  const int l16 = lane & 15, grp = lane >> 4;
  int qrow[NRB];
  bool row_ok[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int lr = 16 * rb + l16;
    qrow[rb] = rt * rpt + lr;
    row_ok[rb] = lr < rpt && qrow[rb] < a.M;
  }

  // Gather rows of this lane: key rows 16 wave + 8 hh + lane / 8 of a tile,
  // 16-byte position lane % 8 of each chunk group (keys past the split end
  // repeat its last key).
  auto slot_of = [&](int t, int hh) {
    int key = k0 + t * SM_NK + wave * 16 + 8 * hh + (lane >> 3);
    key = key < k1 ? key : k1 - 1;
    int64_t si = loc.seg + key;
    si = si < slot_hi ? si : slot_hi;
    return a.slot_idx[si];
  };
  const int ld_elem0 = 8 * ((lane & 7) ^ sm_swz(lane >> 3));
  const int ld_elem1 = 8 * ((lane & 7) ^ sm_swz(8 + (lane >> 3)));
  auto gather_load = [&](int s0, int s1, u32x4 (&gv)[SM_LOADS]) {
    s0 = s0 < 0 ? 0 : (s0 > pool_hi ? pool_hi : s0);
    s1 = s1 < 0 ? 0 : (s1 > pool_hi ? pool_hi : s1);
    const uint16_t* src0 = a.kv + (int64_t)s0 * KV_DIM + ld_elem0;
    const uint16_t* src1 = a.kv + (int64_t)s1 * KV_DIM + ld_elem1;
#pragma unroll
    for (int j = 0; j < CHUNK_GROUPS; ++j) {
      gv[2 * j] = *reinterpret_cast<const u32x4*>(src0 + 64 * j);
      gv[2 * j + 1] = *reinterpret_cast<const u32x4*>(src1 + 64 * j);
    }
  };
  auto gather_store = [&](int t, const u32x4 (&gv)[SM_LOADS]) {
    const uint32_t dst = smem_base + (t & 1) * SM_TILE_BYTES + wave * 16 * 128 + 16 * lane;
#pragma unroll
    for (int j = 0; j < CHUNK_GROUPS; ++j) {
      lds_write_b128(dst + j * SM_GROUP_BYTES, gv[2 * j]);
      lds_write_b128(dst + j * SM_GROUP_BYTES + 8 * 128, gv[2 * j + 1]);
    }
  };

  // ---- prologue, loads oldest first: slot entries of tile 0, the tree's
  // parent pointers (wave 0), the query block, slot entries of tile 1, then
  // the gather of tile 0 once its slot entries are in.
  int sn0 = slot_of(0, 0), sn1 = slot_of(0, 1);
  int parent = -1;
  if (wave == 0) parent = a.tree_parent[(int64_t)loc.b * a.T + (lane < a.T ? lane : a.T - 1)];
  // The query block (the workgroup's 32 local rows, 1,152 bytes each) passes
  // through LDS, in tile 1's buffer, which is free until the end of the first
  // iteration: wave w loads local rows 8w .. 8w+7 with nine 1 KB loads (16-byte
  // piece s of the block holds piece (s % 72) ^ (row % 8) of row s / 72, so that
  // the reads below, eight consecutive rows per cycle, hit distinct banks);
  // rows past the tile read the tile's first row and are zeroed when read.
  const uint32_t qstage = smem_base + SM_TILE_BYTES;
  u32x4 qs[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int sidx = 72 * 8 * wave + 64 * j + lane;
    const int r = sidx / 72, pc = (sidx - 72 * r) ^ (r & 7);
    const int gr = rt * rpt + r;
    const int grow = (r < rpt && gr < a.M) ? gr : rt * rpt;
    qs[j] = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)loc.b * a.M + grow) * KV_DIM + 8 * pc);
  }
  int sx0 = slot_of(1, 0), sx1 = slot_of(1, 1);
  u32x4 gv[SM_LOADS];
  gather_load(sn0, sn1, gv);
#pragma unroll
  for (int j = 0; j < 9; ++j) lds_write_b128(qstage + 1024 * (9 * wave + j) + 16 * lane, qs[j]);
  gather_store(0, gv);
  lds_barrier();  // the query block and tile 0 in LDS
  sn0 = sx0;
  sn1 = sx1;
  // Query fragments (B operand of S^T = K Q^T): lane l holds local row
  // 16 rb + l%16, features 32 ks + 8 (l/16) .. +7 (piece 4 ks + l/16).
  bf16x8 qf[NRB][SM_QK_STEPS];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = 16 * rb + l16;
#pragma unroll
    for (int ks = 0; ks < SM_QK_STEPS; ++ks) {
      u32x4 v = __builtin_bit_cast(u32x4, lds_read_b128(qstage + 16 * (72 * r + ((4 * ks + grp) ^ (r & 7)))));
      if (!row_ok[rb]) v = u32x4{0u, 0u, 0u, 0u};
      qf[rb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Ancestor masks (as in verify_attn_partial_kernel).
  if (wave == 0) {
    int up = (parent >= 0 && parent < lane && lane < a.T) ? parent : -1;
    unsigned long long m = lane < a.T ? (1ull << lane) : 0ull;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int src = up >= 0 ? up : lane;
      const unsigned long long m_up = __shfl(m, src);
      const int up_up = __shfl(up, src);
      if (up >= 0) {
        m |= m_up;
        up = up_up;
      }
    }
    if (lane < a.T) anc_s[lane] = m;
  }

  // Operand read offsets inside a tile (chunk group added per step).
  //  QK step ks: key row 16 wave + l%16, chunk 4 ks + l/16.
  int qk_off[2];
  {
    const int kr = wave * 16 + l16;
#pragma unroll
    for (int h = 0; h < 2; ++h) qk_off[h] = kr * 128 + (((4 * h + grp) ^ sm_swz(kr)) << 4);
  }
  //  PV block fb, key step ks, half h: 16-lane group G = l/16, lane 4r + c of
  //  the group addresses key row 32 ks + 8 G + 4 h + r, features
  //  128 wave + 16 fb + 4c .. +3 (chunk 16 wave + 2 fb + c/2, 8-byte half c%2).
  // (The swizzle of key row kr depends on kr % 16 only, so key step ks adds
  // 32 * 128 bytes.)
  int pv_off[2][4];  // [h][fb % 4] at ks = 0
  {
    const int r = l16 >> 2, c = l16 & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int f4 = 0; f4 < 4; ++f4) {
        const int kr = 8 * grp + 4 * h + r;
        const int pos = (2 * f4 + (c >> 1)) ^ sm_swz(kr);
        pv_off[h][f4] = kr * 128 + (pos << 4) + 8 * (c & 1);
      }
  }
  // Weight block: row lr, keys 8 j .. 8 j + 7 at lr * 128 + ((j ^ sm_swz(lr)) << 4).
  auto p_addr = [&](int lr, int j) { return p_base + lr * 128 + (((j ^ sm_swz(lr)) & 7) << 4); };

  f32x4 o[SM_FB][NRB];
#pragma unroll
  for (int fb = 0; fb < SM_FB; ++fb)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) o[fb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NRB], l_run[NRB];  // running reference max of local row 16 rb + l%16, this lane's share of its sum
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  for (int it = 0; it < ntiles; ++it) {
    // The barrier publishes tile it (written by every wave at the end of the
    // previous iteration, or in the prologue) and frees the other buffer (every
    // wave is done with tile it-1, and, at it = 0, with the query block).
    lds_barrier();
    const uint32_t cur = smem_base + (it & 1) * SM_TILE_BYTES;
    const bool more = it + 1 < ntiles;  // wave-uniform
    if (more) {
      gather_load(sn0, sn1, gv);  // tile it+1, written into LDS after PV
      sx0 = slot_of(it + 2, 0);
      sx1 = slot_of(it + 2, 1);
    }

    // ---- S^T = K Q^T for this wave's 16 keys: lane l holds row 16 rb + l%16,
    // keys 16 wave + 4 (l/16) + i, i < 4 (two accumulators per row block, even
    // and odd k-steps).
    f32x4 s2[NRB][2];
    {
      constexpr int AHEAD = 4;
      auto kread = [&](int ks) { return lds_read_b128(cur + (ks >> 1) * SM_GROUP_BYTES + qk_off[ks & 1]); };
      bf16x8 kbuf[AHEAD];
#pragma unroll
      for (int ks = 0; ks < AHEAD; ++ks) kbuf[ks] = kread(ks);
#pragma unroll
      for (int ks = 0; ks < SM_QK_STEPS; ++ks) {
        const bf16x8 kv = kbuf[ks % AHEAD];
        if (ks + AHEAD < SM_QK_STEPS) kbuf[ks % AHEAD] = kread(ks + AHEAD);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          if (ks < 2) mfma16_qk_first(s2[rb][ks], kv, qf[rb][ks]);
          else mfma16_qk(s2[rb][ks & 1], kv, qf[rb][ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    static_assert(NRB == 1 || NRB == 2, "row blocks");
    mfma_drain_acc<NRB>(s2);  // the QK accumulators are read below
    f32x4 s[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) s[rb] = s2[rb][0] + s2[rb][1];
    // ---- scale, tree mask, the tile's row maxima through LDS
    const int kt = k0 + it * SM_NK;
    const int kb = kt + wave * 16 + 4 * grp;  // key of s[rb][0]
    const bool edge = kt + SM_NK > k1 || kt + SM_NK > P;  // the tile reaches the split end or the tree
    float mx[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[rb][i] *= a.qk_scale_log2;
      if (edge) {
        const unsigned long long anc = anc_s[row_ok[rb] ? qrow[rb] / a.H : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + i;
          const int u = key - P;
          const bool vis = (key < k1) & ((u < 0) | (((anc >> (u & 63)) & 1ull) != 0));
          s[rb][i] = vis ? s[rb][i] : -INFINITY;
        }
      }
      float m4 = fmaxf(fmaxf(s[rb][0], s[rb][1]), fmaxf(s[rb][2], s[rb][3]));
      m4 = fmaxf(m4, xor16(m4));  // the four lane groups hold keys of the same row
      mx[rb] = fmaxf(m4, xor32(m4));
    }
    if (grp == 0) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        *(LDS_AS float*)(uintptr_t)(rmax_base + ((16 * rb + l16) * NWAVES + wave) * 4) = mx[rb];
    }
    lds_barrier();

    // ---- online softmax (every wave takes the same decision per row), the
    // bf16 weights of this wave's keys into the weight block
    bool any_raise = false;
    float alpha[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const f32x4 wm = *(const LDS_AS f32x4*)(uintptr_t)(rmax_base + (16 * rb + l16) * NWAVES * 4);
      const float t = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
      const bool raise = t > m_run[rb] + LAZY_RESCALE_LOG2;
      // O needs rescaling only in rows that already hold weights
      any_raise |= __ballot(raise & (m_run[rb] != -INFINITY)) != 0;
      alpha[rb] = raise ? __builtin_amdgcn_exp2f(m_run[rb] - t) : 1.0f;  // m_run = -inf -> 0
      m_run[rb] = raise ? t : m_run[rb];
      const float mu = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
      bf16x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = (__bf16)__builtin_amdgcn_exp2f(s[rb][i] - mu);
      // the running sum uses the same bf16-rounded weights that enter O
      const u32x2 pbits = __builtin_bit_cast(u32x2, pw);
      l_run[rb] = l_run[rb] * alpha[rb] +
                  ((__builtin_bit_cast(float, pbits[0] << 16) + __builtin_bit_cast(float, pbits[0] & 0xffff0000u)) +
                   (__builtin_bit_cast(float, pbits[1] << 16) + __builtin_bit_cast(float, pbits[1] & 0xffff0000u)));
      {
        const int lr = 16 * rb + l16;
        const int j = 2 * wave + (grp >> 1);  // 8-key piece of keys 16 wave + 4 grp
        *(LDS_AS u32x2*)(uintptr_t)(p_addr(lr, j) + 8 * (grp & 1)) = pbits;
      }
    }
    lds_barrier();

    if (any_raise) {  // O (PV up to tile it-1) *= alpha of its row
#pragma unroll
      for (int fb = 0; fb < SM_FB; ++fb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) o[fb][rb] *= alpha[rb];
    }

    // ---- O^T += V^T P^T: this wave's 8 feature blocks x the rows x 64 keys
    bf16x8 pb[NRB][2];  // [rb][ks]: lane l holds row 16 rb + l%16, keys 32 ks + 8 (l/16) .. +7
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pb[rb][ks] = lds_read_b128(p_addr(16 * rb + l16, 4 * ks + grp));
    {
      auto vread = [&](int st) {  // step st = 8 ks + fb
        const int ks = st >> 3, fb = st & 7;
        const uint32_t base = cur + (2 * wave + (fb >> 2)) * SM_GROUP_BYTES + ks * 32 * 128;
        const bf16x4 v0 = lds_read_tr(base + pv_off[0][fb & 3]);
        const bf16x4 v1 = lds_read_tr(base + pv_off[1][fb & 3]);
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int AHEAD = 4;
      bf16x8 vbuf[AHEAD];
#pragma unroll
      for (int st = 0; st < AHEAD; ++st) vbuf[st] = vread(st);
#pragma unroll
      for (int st = 0; st < 2 * SM_FB; ++st) {
        const bf16x8 vt = vbuf[st % AHEAD];
        if (st + AHEAD < 2 * SM_FB) vbuf[st % AHEAD] = vread(st + AHEAD);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          o[st & 7][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb[rb][st >> 3], o[st & 7][rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) {
      gather_store(it + 1, gv);
      sn0 = sx0;
      sn1 = sx1;
    }
  }

  // ---- partial results: the row's running sum over the four lane groups and
  // the four waves (through the row-max buffer, free since the last barrier),
  // then the split's V average (0 for a row with every key of the split masked)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float t = l_run[rb] + xor16(l_run[rb]);
    t += xor32(t);
    if (grp == 0) *(LDS_AS float*)(uintptr_t)(rmax_base + ((16 * rb + l16) * NWAVES + wave) * 4) = t;
  }
  lds_barrier();
  // The bf16 averages pass through LDS (tile 0's buffer, free since the loop
  // ended): local row lr takes 1 KB, 16-byte chunk c at position c ^ (lr % 64),
  // which spreads a wave's writes (16 rows x two chunks) and the reads of one
  // row evenly over the banks; each row then leaves with one 1 KB store.
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (!row_ok[rb]) continue;
    const f32x4 wl = *(const LDS_AS f32x4*)(uintptr_t)(rmax_base + (16 * rb + l16) * NWAVES * 4);
    const float t = (wl[0] + wl[1]) + (wl[2] + wl[3]);
    const float inv = t > 0.f ? 1.0f / t : 0.f;
    const int lr = 16 * rb + l16;
#pragma unroll
    for (int fb = 0; fb < SM_FB; ++fb) {
      const int c = 16 * wave + 2 * fb + (grp >> 1);  // features 128 wave + 16 fb + 4 grp .. +3
      *(LDS_AS u32x2*)(uintptr_t)(smem_base + lr * (V_DIM * 2) + ((c ^ lr) << 4) + 8 * (grp & 1)) =
          u32x2{pack_bf16x2(o[fb][rb][0] * inv, o[fb][rb][1] * inv),
                pack_bf16x2(o[fb][rb][2] * inv, o[fb][rb][3] * inv)};
    }
    if (wave == 0 && grp == 0) {
      const int64_t rowid = (int64_t)g * a.M + qrow[rb];
      a.part_ml[2 * rowid] = m_run[rb];
      a.part_ml[2 * rowid + 1] = t;
    }
  }
  lds_barrier();
  const int nrows = min(rpt, a.M - rt * rpt);  // valid local rows: 0 .. nrows-1
  uint16_t* po = a.part_o + ((int64_t)g * a.M + rt * rpt) * V_DIM + 8 * lane;
  for (int lr = wave; lr < nrows; lr += NWAVES) {
    const u32x4 v = *(const LDS_AS u32x4*)(uintptr_t)(smem_base + lr * (V_DIM * 2) + ((lane ^ lr) << 4));
    *reinterpret_cast<u32x4*>(po + (int64_t)lr * V_DIM) = v;
  }
}


__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void verify_attn_f32_partial_kernel(PartialF32Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[F_NBUF * F_TILE_BYTES];
  __shared__ unsigned long long anc_s[MAX_TREE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int g, rt;
  SplitLoc loc;
  if (!locate_item(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, a.max_splits, a.row_tiles, a.nxcd, &g, &rt, &loc)) return;
  g = __builtin_amdgcn_readfirstlane(g);
  rt = __builtin_amdgcn_readfirstlane(rt);
  loc.b = __builtin_amdgcn_readfirstlane(loc.b);
  loc.len = __builtin_amdgcn_readfirstlane(loc.len);
  loc.seg = ((int64_t)__builtin_amdgcn_readfirstlane((int)(loc.seg >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)loc.seg);
  const int k0 = (g - __builtin_amdgcn_readfirstlane(loc.g0)) * a.chunk;
  const int k1 = min(k0 + a.chunk, loc.len);
  const int P = loc.len - a.T;
  const int ntiles = (k1 - k0 + F_NK - 1) / F_NK;
  const uint32_t smem_base = lds_addr(smem);
  const int64_t slot_hi = a.total_kv - 1;
  const int pool_hi = (int)(a.pool_slots - 1 < (int64_t)INT32_MAX ? a.pool_slots - 1 : (int64_t)INT32_MAX);
  const int grp = lane >> 4;  // reduction lane group
  const int l16 = lane & 15;

  // Gather of one tile: load j, lane -> LDS byte 1024 j + 16 lane of this
  // wave's 4-row band -> (row, position) -> piece position ^ (row % 16).
  int g_row[F_LOADS], g_piece[F_LOADS];
#pragma unroll
  for (int j = 0; j < F_LOADS; ++j) {
    const int o = j * 1024 + 16 * lane;
    const int lr = o / F_ROW_BYTES;
    const int r = wave * (F_NK / NWAVES) + lr;
    g_row[j] = lr;
    g_piece[j] = ((o - lr * F_ROW_BYTES) >> 4) ^ (r & 15);
  }
  // Slot-table entries of this wave's 4-row band of the tile at key kt, as one
  // vector load: lane l reads the entry of row l % 4 (keys past the split end
  // repeat its last key). band_slots() clamps them and reads them out to
  // wave-uniform values where the gather needs them, a tile after the load, so
  // that its round trip overlaps the work in between (four scalar loads, each
  // waited for before the next, would stall the wave four round trips).
  auto band_load = [&](int kt) {
    int key = kt + wave * (F_NK / NWAVES) + (lane & 3);
    key = key < k1 ? key : k1 - 1;
    int64_t si = loc.seg + key;
    si = si < slot_hi ? si : slot_hi;
    return a.slot_idx[si];
  };
  auto band_slots = [&](int v, int (&out)[4]) {
    const int slot = v < 0 ? 0 : (v > pool_hi ? pool_hi : v);
#pragma unroll
    for (int lr = 0; lr < 4; ++lr) out[lr] = __builtin_amdgcn_readlane(slot, lr);
  };
  auto gather_one = [&](int t, const int (&slots)[4], int j) {  // load j of tile t
    const uint32_t dst = smem_base + (t % F_NBUF) * F_TILE_BYTES + wave * (F_NK / NWAVES) * F_ROW_BYTES;
    const int lr = g_row[j];
    const int slot = lr == 0 ? slots[0] : (lr == 1 ? slots[1] : (lr == 2 ? slots[2] : slots[3]));
    load_to_lds16(a.kv + (int64_t)slot * KV_DIM + 4 * g_piece[j], dst + j * 1024);
  };
  auto gather = [&](int t, const int (&slots)[4]) {
#pragma unroll
    for (int j = 0; j < F_LOADS; ++j) gather_one(t, slots, j);
  };

  // Prologue: parent pointers, the slots and gathers of tiles 0 and 1, the
  // query fragments, the ancestor masks.
  int parent = -1;
  if (wave == 0 && lane < a.T) parent = a.tree_parent[(int64_t)loc.b * a.T + lane];
  {
    const int v0 = band_load(k0), v1 = band_load(k0 + F_NK);
    int s0[4], s1[4];
    band_slots(v0, s0);
    band_slots(v1, s1);
    gather(0, s0);
    gather(1, s1);
  }
  const int row0 = rt * F_ROWS_PER_TILE + wave * F_ROWS_PER_WAVE;
  const bool wave_active = row0 < a.M;
  const int qrow = row0 + l16;
  const bool row_ok = qrow < a.M;
  f32x4 qf[F_CHUNKS];
  {
    const float* src = a.q + ((int64_t)loc.b * a.M + (row_ok ? qrow : 0)) * KV_DIM + 4 * grp;
#pragma unroll
    for (int c = 0; c < F_CHUNKS; ++c) {
      f32x4 v = *reinterpret_cast<const f32x4*>(src + 16 * c);
      qf[c] = row_ok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (wave == 0) {  // ancestor masks by pointer jumping (as in the bf16 kernel)
    int up = (parent >= 0 && parent < lane && lane < a.T) ? parent : -1;
    unsigned long long m = lane < a.T ? (1ull << lane) : 0ull;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int src = up >= 0 ? up : lane;
      const unsigned long long m_up = __shfl(m, src);
      const int up_up = __shfl(up, src);
      if (up >= 0) {
        m |= m_up;
        up = up_up;
      }
    }
    if (lane < a.T) anc_s[lane] = m;
  }

  // K read (chunk c): lane (key l16, group grp) reads piece 4c + grp of key
  // row l16, stored at position (4c + grp) ^ l16 = 16 (c / 4) + 4 ((c % 4) ^ (l16 / 4))
  // + (grp ^ (l16 % 4)): a per-lane base for each c % 4 plus 256 (c / 4).
  uint32_t k_off[4];
#pragma unroll
  for (int c3 = 0; c3 < 4; ++c3)
    k_off[c3] = l16 * F_ROW_BYTES + ((((c3 ^ (l16 >> 2)) << 2) | (grp ^ (l16 & 3))) << 4);
  // V read (key step i, block group J): lane (m = l16, group grp) reads piece
  // 16 J + l16 of key row r = 4 grp + i (features 64 J + 4 l16 .. +3), stored at
  // position 16 J + (l16 ^ r % 16): a per-lane base for each i plus 256 J.
  uint32_t v_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v_off[i] = (4 * grp + i) * F_ROW_BYTES + ((l16 ^ ((4 * grp + i) & 15)) << 4);
  f32x4 o[F_PV_BLOCKS];
#pragma unroll
  for (int e = 0; e < F_PV_BLOCKS; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  int slot_pre = band_load(2 < ntiles ? k0 + 2 * F_NK : k0);  // slot entries of tile 2
  for (int it = 0; it < ntiles; ++it) {
    wait_vmcnt<0>();  // own share of tile it (and of it+1) landed
    lds_barrier();    // tile it complete; every wave is done with tile it-1
    const uint32_t cur = smem_base + (it % F_NBUF) * F_TILE_BYTES;
    const int kt = k0 + it * F_NK;
    // The gather of tile it+2 rides on this QK, one load every two chunks (a
    // burst of nine loads stalls the wave for most of their issue); its slot
    // entries were loaded during tile it-1, and those of tile it+3 go out now.
    const bool more = it + 2 < ntiles;
    const int slot_next = slot_pre;
    slot_pre = band_load(it + 3 < ntiles ? kt + 3 * F_NK : kt);
    int sn[4] = {0, 0, 0, 0};
    // ---- S^T = K Q^T: 36 chunks x 4 MFMAs, two accumulators (even / odd k-steps)
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    uint32_t kb[4];  // per-tile bases; chunk c reads kb[c % 4] + 256 (c / 4)
#pragma unroll
    for (int c3 = 0; c3 < 4; ++c3) kb[c3] = cur + k_off[c3];
    auto kread = [&](int c) { return *(const LDS_AS f32x4*)(uintptr_t)(kb[c & 3] + 256 * (c >> 2)); };
    constexpr int FK_AHEAD = 4;  // K reads in flight
    f32x4 kbuf[FK_AHEAD];
#pragma unroll
    for (int c = 0; c < FK_AHEAD; ++c) kbuf[c] = kread(c);
#pragma unroll
    for (int c = 0; c < F_CHUNKS; ++c) {
      const f32x4 kv = kbuf[c % FK_AHEAD];
      if (c + FK_AHEAD < F_CHUNKS) kbuf[c % FK_AHEAD] = kread(c + FK_AHEAD);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[i], qf[c][i], sacc[i & 1], 0, 0, 0);
      if (more && c == 1) band_slots(slot_next, sn);
      if (more && c >= 2 && (c - 2) % 2 == 0 && (c - 2) / 2 < F_LOADS) gather_one(it + 2, sn, (c - 2) / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- scale, mask, online softmax (base 2); lane: row l16, keys 4 grp + i
    const unsigned long long anc_row = anc_s[row_ok ? qrow / a.H : 0];
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt + 4 * grp + i;
      const int u = key - P;
      const bool vis = (key < k1) & ((u < 0) | (((anc_row >> (u & 63)) & 1ull) != 0));
      sv[i] = vis ? (sacc[0][i] + sacc[1][i]) * a.qk_scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, xor16(mx));  // the four lane groups hold keys of the same row
    mx = fmaxf(mx, xor32(mx));
    const bool raise = mx > m_run + LAZY_RESCALE_LOG2;
    const bool rescale = __ballot(raise & (m_run != -INFINITY)) != 0;  // rows with weights so far
    const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
    m_run = raise ? mx : m_run;
    const float mu = m_run == -INFINITY ? 0.f : m_run;
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
    l_run = l_run * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
    if (rescale) {  // O (PV up to tile it-1) *= alpha
      mfma_drain();
#pragma unroll
      for (int e = 0; e < F_PV_BLOCKS; ++e) acc_scale4(o[e], alpha);
      mfma_valu_gap();
    }
    // ---- O^T += V^T P^T: 4 key steps x 8 block groups x 4 blocks, one 16-byte
    // V read per group (consecutive MFMAs use different accumulators)
    mfma_valu_gap();
    uint32_t vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vb[i] = cur + v_off[i];
    auto vread = [&](int st) {  // step st = 8 i + J
      return *(const LDS_AS f32x4*)(uintptr_t)(vb[st >> 3] + 256 * (st & 7));
    };
    constexpr int V_AHEAD = 3;  // V reads in flight (more spill registers)
    f32x4 vbuf[V_AHEAD];
#pragma unroll
    for (int st = 0; st < V_AHEAD; ++st) vbuf[st] = vread(st);
#pragma unroll
    for (int st = 0; st < F_PV_BLOCKS; ++st) {
      const f32x4 v = vbuf[st % V_AHEAD];
      if (st + V_AHEAD < F_PV_BLOCKS) vbuf[st % V_AHEAD] = vread(st + V_AHEAD);
      const int J = st & 7;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) mfma16_acc(o[4 * J + e4], v[e4], pw[st >> 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // no gather lands in LDS after this
  mfma_drain();
  lds_barrier();    // every wave is done with the tile buffers, which now stage the partial rows

  if (!wave_active) return;
  // l: the four lane groups of a row hold disjoint keys
  float l_row = l_run + __shfl_xor(l_run, 16);
  l_row += __shfl_xor(l_row, 32);
  // The split's V average (0 for a row with every key of the split masked)
  // leaves through LDS in two halves of 256 features: the wave's 16 rows take
  // 1 KB each (16-byte chunk c at position c ^ row), and each row half then
  // leaves with one contiguous 1 KB store.
  const float inv = (row_ok && l_row > 0.f) ? 1.0f / l_row : 0.f;
  const uint32_t stage = smem_base + wave * (F_ROWS_PER_WAVE * 1024);
  const int nrows = min(F_ROWS_PER_WAVE, a.M - row0);  // wave-uniform, >= 1
  float* po = a.part_o + ((int64_t)g * a.M + row0) * V_DIM + 4 * lane;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int J = 4 * half; J < 4 * half + 4; ++J)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // features 64 J + 16 grp + 4 j .. +3: chunk c of the half
        const int c = 16 * (J - 4 * half) + 4 * grp + j;
        *(LDS_AS f32x4*)(uintptr_t)(stage + l16 * 1024 + ((c ^ l16) << 4)) =
            f32x4{o[4 * J][j], o[4 * J + 1][j], o[4 * J + 2][j], o[4 * J + 3][j]} * inv;
      }
    for (int r = 0; r < nrows; ++r) {
      const f32x4 v = *(const LDS_AS f32x4*)(uintptr_t)(stage + r * 1024 + ((lane ^ r) << 4));
      *reinterpret_cast<f32x4*>(po + (int64_t)r * V_DIM + 256 * half) = v;
    }
  }
  if (row_ok && grp == 0) {
    const int64_t rowid = (int64_t)g * a.M + qrow;
    a.part_ml[2 * rowid] = m_run;
    a.part_ml[2 * rowid + 1] = l_row;
  }
}

// ------------------------------------------------------------ combine kernel
// Output row (b, r) = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s over
// the sequence's splits s (o_s the split's V average, l_s its running sum,
// m_s its running maximum), M = max_s m_s, rounded to bf16 (nearest even).
// WPR waves share one row: wave k reduces splits k, k + WPR, ... in order, and
// the WPR wave results are merged in wave order through LDS, so the result
// does not depend on timing. A wave takes its splits a batch at a time
// (COMBINE_BATCH, _HALF or _F32 of them) with every load of the
// batch issued before the first use (one memory round trip per batch),
// keeping a running maximum and rescaling its sums when the maximum rises.
// The V averages o_s are bf16 on the bf16 path (lane j covers features
// 8j .. 8j+7: one 16-byte load per partial row and lane) and fp32 on the
// fp32-input path (F32_OUT; lane j covers 4j .. 4j+3 and 256 + 4j .. +3).
// HALF: two workgroups per row group, one per half of the 512 features (lane
// j then covers 4j .. 4j+3 of its half).
template <int WPR, bool F32_OUT, bool HALF = false>
__global__ __launch_bounds__((WPR < 4 ? 4 : WPR) * 64) void verify_attn_combine_kernel(CombineArgs a) {
  constexpr int WAVES = WPR < 4 ? 4 : WPR;
  constexpr int ROWS = WAVES / WPR;
  constexpr int BATCH = F32_OUT ? COMBINE_BATCH_F32 : (HALF ? COMBINE_BATCH_HALF : COMBINE_BATCH);
  __shared__ float red_ml[WAVES][2];
  __shared__ f32x4 red_o[WPR > 1 ? WAVES : 1][2 * 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = wave % WPR;
  const int64_t grow = (int64_t)(HALF ? blockIdx.x >> 1 : blockIdx.x) * ROWS + wave / WPR;
  // first feature of this lane (acc0); acc1 holds the next four (bf16
  // partials) or the four 256 further on (fp32 partials)
  const int foff = HALF ? (blockIdx.x & 1) * 256 + 4 * lane : (F32_OUT ? 4 * lane : 8 * lane);
  const bool active = grow < (int64_t)a.B * a.M;
  const int b = active ? (int)(grow / a.M) : 0;
  const int row = active ? (int)(grow - (int64_t)b * a.M) : 0;

  // One batch: partials base + j * WPR (j < BATCH) below `limit`, as loaded
  // (ra: the V average's bits at foff; rb: fp32 at foff + 256). Entries at or
  // past the limit are left unloaded and never read.
  f32x2 ml[BATCH];
  u32x4 ra[BATCH];
  u32x4 rb[F32_OUT && !HALF ? BATCH : 1];
  auto load = [&](int base, int limit) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (base + j * WPR >= limit) continue;  // wave-uniform
      const int64_t rowid = (int64_t)(base + j * WPR) * a.M + row;
      ml[j] = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * rowid);
      if constexpr (F32_OUT) {
        const float* src = static_cast<const float*>(a.part_o) + rowid * V_DIM + foff;
        ra[j] = *reinterpret_cast<const u32x4*>(src);
        if constexpr (!HALF) rb[j] = *reinterpret_cast<const u32x4*>(src + 256);
      } else if constexpr (HALF) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.part_o) + rowid * V_DIM + foff);
        ra[j] = u32x4{w[0], w[1], 0u, 0u};
      } else {
        ra[j] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.part_o) + rowid * V_DIM + foff);
      }
    }
  };

  // Sequence 0's splits start at global split 0, so its rows issue their first
  // batch (bounded by max_splits, inside the workspace) before the split count
  // is known; every other row locates its sequence's splits first.
  const bool first_seq = active && b == 0;
  int g0 = 0, g_end = 0;
  if (first_seq) {
    load(sub, a.max_splits);
    const int len = clamp_len(a.seq_lens[0], a.T, a.max_seq_len);
    g_end = (len + a.chunk - 1) / a.chunk;
  } else if (active) {
    SplitLoc loc;
    if (locate_split(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, b, true, &loc)) {
      g0 = loc.g0;
      g_end = loc.g0 + loc.n_splits;
    }
  }
  g_end = g_end < a.max_splits ? g_end : a.max_splits;
  int base = g0 + sub;
  if (!first_seq && base < g_end) load(base, g_end);

  float mloc = -INFINITY;  // running maximum of this wave's splits
  float L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  while (base < g_end) {
    float mb = mloc;
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (base + j * WPR < g_end) mb = fmaxf(mb, ml[j][0]);
    if (mb > mloc) {  // the same for every lane (one row per wave)
      const float s = exp2f(mloc - mb);  // mloc = -inf -> 0
      acc0 *= s;
      acc1 *= s;
      L *= s;
      mloc = mb;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (base + j * WPR >= g_end || ml[j][0] == -INFINITY) continue;  // wave-uniform
      const float w = exp2f(ml[j][0] - mloc) * ml[j][1];
      f32x4 o0, o1;
      if constexpr (F32_OUT) {
        o0 = __builtin_bit_cast(f32x4, ra[j]);
        o1 = HALF ? f32x4{0.f, 0.f, 0.f, 0.f} : __builtin_bit_cast(f32x4, rb[HALF ? 0 : j]);
      } else {
        o0 = f32x4{bf16_lo(ra[j][0]), bf16_hi(ra[j][0]), bf16_lo(ra[j][1]), bf16_hi(ra[j][1])};
        o1 = HALF ? f32x4{0.f, 0.f, 0.f, 0.f}
                  : f32x4{bf16_lo(ra[j][2]), bf16_hi(ra[j][2]), bf16_lo(ra[j][3]), bf16_hi(ra[j][3])};
      }
      acc0 += w * o0;
      acc1 += w * o1;
      L += w;
    }
    base += WPR * BATCH;
    if (base < g_end) load(base, g_end);
  }

  if constexpr (WPR > 1) {
    if (lane == 0) {
      red_ml[wave][0] = mloc;
      red_ml[wave][1] = L;
    }
    red_o[wave][2 * lane] = acc0;
    red_o[wave][2 * lane + 1] = acc1;
    __syncthreads();
    if (sub != 0) return;
    float mm = -INFINITY;
    for (int k = 0; k < WPR; ++k) mm = fmaxf(mm, red_ml[wave + k][0]);
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    L = 0.f;
    for (int k = 0; k < WPR; ++k) {
      const float mk = red_ml[wave + k][0];
      const float w = (mk == -INFINITY) ? 0.f : exp2f(mk - mm);
      acc0 += w * red_o[wave + k][2 * lane];
      acc1 += w * red_o[wave + k][2 * lane + 1];
      L += w * red_ml[wave + k][1];
    }
  }
  if (!active) return;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  if constexpr (F32_OUT) {
    float* dst = a.out_f32 + grow * V_DIM + foff;
    *reinterpret_cast<f32x4*>(dst) = acc0;
    if (!HALF) *reinterpret_cast<f32x4*>(dst + 256) = acc1;
  } else {
    uint16_t* dst = a.out + grow * V_DIM + foff;
    const u32x2 p0 = {pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3])};
    if (HALF)
      *reinterpret_cast<u32x2*>(dst) = p0;
    else
      *reinterpret_cast<u32x4*>(dst) = u32x4{p0[0], p0[1], pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
  }
}

// Combine for few rows (bf16 partials): one workgroup per (row, 64-feature
// slice), so that a call with few rows still spreads the partial reads over
// the device's CUs (each CU fetches rows of partials at a bounded rate). The
// arithmetic is that of verify_attn_combine_kernel. Lane l reads features
// 4 (l % 16) .. +3 of the slice (8 bytes) of split 4 (W j + w) + l / 16 of the
// batch, so one load instruction covers four splits' 128-byte segments; wave
// w takes splits 4 w .. 4 w + 3, 4 (W + w) .. of each batch of 4 W
// COMBINE_BATCH_SLICE splits. Every lane keeps a running maximum, sum and four
// feature sums over its own splits; the four lanes of a feature group are
// then merged (lane xor 16, then xor 32: both lanes of a pair compute the same
// products and sums, in commuted order, so they agree exactly) and the W waves'
// results in wave order through LDS. Deterministic: the order depends only on
// the plan.
template <int W>
__global__ __launch_bounds__(W * 64) void verify_attn_combine_slice_kernel(CombineArgs a) {
  constexpr int BATCH = COMBINE_BATCH_SLICE;
  __shared__ float red[W][16][6];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t grow = blockIdx.x / COMBINE_SLICES;
  const int foff = (blockIdx.x % COMBINE_SLICES) * 64 + 4 * (lane & 15);
  const int sl = lane >> 4;
  if (grow >= (int64_t)a.B * a.M) return;  // workgroup-uniform
  const int b = (int)(grow / a.M);
  const int row = (int)(grow - (int64_t)b * a.M);
  const uint16_t* part_o = static_cast<const uint16_t*>(a.part_o);

  // One batch from split `first` (the lane's own first split): splits
  // first + 4 W j, those at or past `limit` replaced by limit - 1 (loaded,
  // never used): unconditional loads keep the compiler's waits per batch.
  f32x2 ml[BATCH];
  u32x2 ra[BATCH];
  auto load = [&](int first, int limit) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int sp = min(first + 4 * W * j, limit - 1);
      const int64_t rowid = (int64_t)sp * a.M + row;
      ml[j] = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * rowid);
      ra[j] = *reinterpret_cast<const u32x2*>(part_o + rowid * V_DIM + foff);
    }
  };

  // Sequence 0's splits start at global split 0: its rows issue their first
  // batch (bounded by max_splits, inside the workspace) before the split
  // count is known; every other row locates its sequence's splits first.
  int g0 = 0, g_end = 0;
  if (b == 0) {
    load(4 * wave + sl, a.max_splits);
    const int len = clamp_len(a.seq_lens[0], a.T, a.max_seq_len);
    g_end = (len + a.chunk - 1) / a.chunk;
  } else {
    SplitLoc loc;
    if (locate_split(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, b, true, &loc)) {
      g0 = loc.g0;
      g_end = loc.g0 + loc.n_splits;
    }
  }
  g_end = g_end < a.max_splits ? g_end : a.max_splits;
  int first = g0 + 4 * wave + sl;
  if (b != 0 && g0 + 4 * wave < g_end) load(first, g_end);  // wave-uniform

  float mloc = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // wave-uniform loop bound: the wave's first split of the batch
  for (int wbase = g0 + 4 * wave; wbase < g_end; wbase += 4 * W * BATCH) {
    float mb = mloc;
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (first + 4 * W * j < g_end) mb = fmaxf(mb, ml[j][0]);
    if (mb > mloc) {
      const float sc = exp2f(mloc - mb);  // mloc = -inf -> 0
      acc *= sc;
      L *= sc;
      mloc = mb;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (first + 4 * W * j >= g_end || ml[j][0] == -INFINITY) continue;
      const float w = exp2f(ml[j][0] - mloc) * ml[j][1];
      acc += w * f32x4{bf16_lo(ra[j][0]), bf16_hi(ra[j][0]), bf16_lo(ra[j][1]), bf16_hi(ra[j][1])};
      L += w;
    }
    first += 4 * W * BATCH;
    if (wbase + 4 * W * BATCH < g_end) load(first, g_end);
  }

  // (m, L, acc) of two lanes or waves merged under their common maximum.
  auto merge = [&](float m_o, float L_o, const f32x4& acc_o) {
    const float mm = fmaxf(mloc, m_o);
    const float s0 = mloc == -INFINITY ? 0.f : exp2f(mloc - mm);
    const float s1 = m_o == -INFINITY ? 0.f : exp2f(m_o - mm);
    acc = acc * s0 + acc_o * s1;
    L = L * s0 + L_o * s1;
    mloc = mm;
  };
#pragma unroll
  for (int d = 16; d <= 32; d *= 2) {
    const float m_o = __shfl_xor(mloc, d);
    const float L_o = __shfl_xor(L, d);
    f32x4 acc_o;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc_o[k] = __shfl_xor(acc[k], d);
    merge(m_o, L_o, acc_o);
  }
  if constexpr (W > 1) {
    if (lane < 16) {
      red[wave][lane][0] = mloc;
      red[wave][lane][1] = L;
#pragma unroll
      for (int k = 0; k < 4; ++k) red[wave][lane][2 + k] = acc[k];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < W; ++w)
      merge(red[w][lane & 15][0], red[w][lane & 15][1],
            f32x4{red[w][lane & 15][2], red[w][lane & 15][3], red[w][lane & 15][4], red[w][lane & 15][5]});
  }
  if (lane >= 16) return;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  acc *= inv;
  *reinterpret_cast<u32x2*>(a.out + grow * V_DIM + foff) =
      u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
}

// ------------------------------------------------------------ append kernel
// Draft-row KV append: row (b, t) of kv_new -> kv_pool[slot of tree node t of
// sequence b] (the last T entries of the sequence's slot_idx segment). One
// wave per row: 64 lanes copy 1,024 bytes, lanes 0..7 the last 128.
__global__ __launch_bounds__(256) void verify_attn_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * T + t
  if (r >= (int64_t)a.B * a.T) return;
  const int b = (int)(r / a.T);
  const int t = (int)(r - (int64_t)b * a.T);
  long long seg = 0;  // segment start: sum of the (clamped) lengths of sequences < b
  for (int bb = lane; bb < b; bb += 64) seg += clamp_len(a.seq_lens[bb], a.T, a.max_seq_len);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) seg += __shfl_xor(seg, d);
  int64_t si = seg + clamp_len(a.seq_lens[b], a.T, a.max_seq_len) - a.T + t;
  si = si < a.total_kv - 1 ? si : a.total_kv - 1;
  const int slot = a.slot_idx[si];
  if (slot < 0 || (int64_t)slot >= a.pool_slots) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.kv_new + r * KV_DIM);
  u32x4* dst = reinterpret_cast<u32x4*>(a.kv_pool + (int64_t)slot * KV_DIM);
  dst[lane] = src[lane];
  if (lane < 8) dst[64 + lane] = src[64 + lane];
}

// ------------------------------------------------------------ compact kernel
// KV defragmentation: kv_dst[i] = kv_pool[slot_idx[i]]. One wave per row, four
// rows per workgroup; 16 bytes per lane (the last 128 bytes on lanes 0..7).
__global__ __launch_bounds__(256) void verify_attn_compact_kernel(CompactArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= a.total_kv) return;
  const int slot = a.slot_idx[i];
  u32x4* dst = reinterpret_cast<u32x4*>(a.kv_dst + i * KV_DIM);
  if (slot < 0 || (int64_t)slot >= a.pool_slots) {
    dst[lane] = u32x4{0u, 0u, 0u, 0u};
    if (lane < 8) dst[64 + lane] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(a.kv_pool + (int64_t)slot * KV_DIM);
  const u32x4 v0 = src[lane];
  u32x4 v1 = {0u, 0u, 0u, 0u};
  if (lane < 8) v1 = src[64 + lane];
  dst[lane] = v0;
  if (lane < 8) dst[64 + lane] = v1;
}

// ------------------------------------------------------------ validation
// Debug check of the device-resident inputs (not on the hot path): bits of
// *flags are set for lengths outside [T, max_seq_len], lengths that add up to
// more than total_kv, parents outside [-1, t-1], slots outside the pool.
struct ValidateArgs {
  const int32_t* slot_idx;
  const int32_t* seq_lens;
  const int32_t* tree_parent;
  int32_t* flags;
  int B, T, max_seq_len;
  int64_t total_kv, pool_slots;
};

__global__ __launch_bounds__(64) void verify_attn_validate_clear(int32_t* flags) {
  if (threadIdx.x == 0) *flags = 0;
}

__global__ __launch_bounds__(256) void verify_attn_validate_kernel(ValidateArgs a) {
  int bits = 0;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * 256;
  if (blockIdx.x == 0 && threadIdx.x < 64) {  // lengths and their sum: one wave
    long long sum = 0;
    for (int b = threadIdx.x; b < a.B; b += 64) {
      const int n = a.seq_lens[b];
      if (n < a.T || n > a.max_seq_len) bits |= VERIFY_ATTN_BAD_LENGTH;
      sum += n;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
    if (sum > a.total_kv) bits |= VERIFY_ATTN_BAD_TOTAL;
  }
  for (int64_t i = gid; i < (int64_t)a.B * a.T; i += nthreads) {
    const int t = (int)(i % a.T);
    const int p = a.tree_parent[i];
    if (p < -1 || p >= t) bits |= VERIFY_ATTN_BAD_PARENT;
  }
  for (int64_t i = gid; i < a.total_kv; i += nthreads) {
    const int slot = a.slot_idx[i];
    if (slot < 0 || (int64_t)slot >= a.pool_slots) bits |= VERIFY_ATTN_BAD_SLOT;
  }
  if (bits) atomicOr(a.flags, bits);
}

// ------------------------------------------------------------------- host

constexpr int MI355X_CUS = 256;     // compute units of a whole MI355X (the plan's default)
constexpr int MI355X_XCDS = 8;      // and its XCDs
constexpr int64_t COMBINE_WAVES_PER_CU = 16;  // combine waves resident at once per CU
constexpr int64_t ROUND_COST_TILES = 4;  // fixed cost of a round of workgroups, in tiles

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate(const verify_attn_params* p) {
  if (!p) return VERIFY_ATTN_ERR_NULL_PTR;
  if (p->num_seqs < 1 || p->num_heads < 1 || p->kv_dim != KV_DIM || p->v_dim != V_DIM ||
      p->page_size < 1 || p->pool_slots < 1 || p->reserved != 0 || !std::isfinite(p->sm_scale))
    return VERIFY_ATTN_ERR_BAD_DIM;
  if (p->tree_size < 1 || p->tree_size > MAX_TREE) return VERIFY_ATTN_ERR_TREE_TOO_LARGE;
  if ((int64_t)p->num_heads * p->tree_size > (1 << 20)) return VERIFY_ATTN_ERR_BAD_DIM;
  if (p->max_seq_len < p->tree_size) return VERIFY_ATTN_ERR_BAD_SEQ;
  if (p->total_kv < (int64_t)p->num_seqs * p->tree_size) return VERIFY_ATTN_ERR_BAD_SEQ;
  if (p->total_kv > (int64_t)p->num_seqs * p->max_seq_len) return VERIFY_ATTN_ERR_BAD_SEQ;
  if (p->nsplit < 0) return VERIFY_ATTN_ERR_BAD_SPLIT;
  return VERIFY_ATTN_OK;
}

// Compute units and XCDs the launch is planned for.
struct DevShape {
  int cus, xcds;
};

// The shape of the current device (its multiProcessorCount: fewer than 256
// under a CU-partitioned mode, and its XCD count), read once per device id and
// cached (thread-safe: a cache entry only ever goes from unknown to a fixed
// value). Without a current device, a whole MI355X.
DevShape current_shape() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return {MI355X_CUS, MI355X_XCDS};
  static long long cache[64];  // 0 unknown, else (cus << 16) | xcds
  long long c = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
  if (!c) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return {MI355X_CUS, MI355X_XCDS};
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 ||
        xcds > cus)
      xcds = 1;
    c = ((long long)cus << 16) | xcds;
    __atomic_store_n(&cache[dev], c, __ATOMIC_RELEASE);
  }
  return {(int)(c >> 16), (int)(c & 0xffff)};
}

// rows_per_tile = 0: the bf16 path, which takes the small-row kernel (at most
// 32 rows per workgroup, 64-key tiles) for H*T <= SM_MAX_M and the 128-row
// kernel otherwise; the fp32 path passes its own geometry.
int make_plan(const verify_attn_params* p, Plan* pl, DevShape dv, int rows_per_tile = 0, int nk = NK) {
  const int rc = validate(p);
  if (rc) return rc;
  if (dv.cus < 1 || dv.xcds < 1 || dv.xcds > dv.cus || dv.cus > (1 << 16)) return VERIFY_ATTN_ERR_BAD_DIM;
  const int64_t NUM_CUS = dv.cus;
  const int64_t M = (int64_t)p->num_heads * p->tree_size;
  const bool bf16_path = rows_per_tile == 0;
  if (rows_per_tile == 0) {
    if (M <= SM_MAX_M) {
      // the rows spread evenly over ceil(M / 32) row tiles
      rows_per_tile = (int)ceil_div64(M, ceil_div64(M, SM_ROWS));
      nk = SM_NK;
    } else {
      rows_per_tile = ROWS_PER_TILE;
      nk = NK;
    }
  }
  const int64_t row_tiles = ceil_div64(M, rows_per_tile);
  int64_t chunk;
  if (p->nsplit > 0) {
    chunk = ceil_div64(p->max_seq_len, p->nsplit);
  } else {
    // For R = 1, 2, ... rounds of one workgroup per CU, take the shortest split
    // (a multiple of nk, at least one tile) whose item count fits R rounds
    // whatever the lengths are: with total_kv keys over num_seqs sequences there
    // are at most ceil(total_kv / c) + num_seqs - 1 splits. Keep the split with
    // the lowest estimated time, in units of one tile of nk keys: every round
    // costs its tiles plus a fixed start and end (about four tiles: first loads,
    // partial store), and every (split, row tile) item about a twentieth of a
    // tile of partial traffic (written, then read by the combine). More, shorter
    // splits fill the last round better but add fixed costs and partials.
    const int64_t split_cap = ceil_div64(p->max_seq_len, nk) * nk;  // one split per sequence
    // The 128-row kernel also tries longer splits (up to 4x) for each round
    // count: its workgroups each stage 147 KB of query and store 128 rows of
    // partials, so fewer, longer splits can win within the same rounds. The
    // small-row kernel's items are cheap, and its shortest split measured best.
    const int64_t widen = (bf16_path && rows_per_tile == ROWS_PER_TILE) ? 4 : 1;
    const int64_t floor_c = nk;
    // fewest rounds with room for every sequence's last split
    const int64_t r0 = ceil_div64((int64_t)p->num_seqs * row_tiles, NUM_CUS);
    int64_t best = 0, best_cost = INT64_MAX;
    for (int64_t R = r0 < 1 ? 1 : r0; R < r0 + 64; ++R) {
      const int64_t splits = NUM_CUS * R / row_tiles - (p->num_seqs - 1);
      if (splits < 1) continue;
      int64_t c = ceil_div64(p->total_kv, splits);
      c = ceil_div64(c, nk) * nk;
      if (c > split_cap) c = split_cap;
      for (int64_t cc = c; cc <= widen * c && cc <= split_cap; cc += nk) {
        const int64_t items = (ceil_div64(p->total_kv, cc) + p->num_seqs - 1) * row_tiles;
        const int64_t cost = ceil_div64(items, NUM_CUS) * (20 * (cc / nk) + 20 * ROUND_COST_TILES) + items;
        if (cost < best_cost) {
          best_cost = cost;
          best = cc;
        }
      }
      if (c <= floor_c) break;  // more rounds cannot shorten the split further
    }
    chunk = best;
  }
  chunk = ceil_div64(chunk, nk) * nk;
  const int64_t len_cap = ceil_div64(p->max_seq_len, nk) * nk;
  if (chunk > len_cap) chunk = len_cap;
  const int64_t max_splits = ceil_div64(p->total_kv, chunk) + p->num_seqs;
  const int64_t blocks = ceil_div64(max_splits * row_tiles, dv.xcds) * dv.xcds;
  // Combine: waves per row (a power of two up to 16, no more than the row's
  // splits) so that all rows' waves fit in about one round of the chip
  // (COMBINE_WAVES), each wave taking its splits in batches of COMBINE_BATCH.
  const int64_t rows = (int64_t)p->num_seqs * M;
  const int64_t seq_splits = ceil_div64(p->max_seq_len, chunk);
  int wpr = 1;
  const int64_t COMBINE_WAVES = COMBINE_WAVES_PER_CU * NUM_CUS;
  while (wpr < 16 && rows * wpr * 2 <= COMBINE_WAVES && wpr * 2 <= seq_splits) wpr *= 2;
  // Few rows: split the features of a row over several workgroups, so that
  // more CUs read the partials. Up to one row per 8 CUs on the bf16 path: the
  // sliced combine (eight 64-feature slices, with the fewest waves, a power of
  // two up to 16, that take a row's splits in one batch); with more rows it
  // measured no faster, and at 128 or more rows slower. Else feature halves.
  int halves = (wpr == 16 && rows * 16 * 2 <= COMBINE_WAVES) ? 2 : 1;
  int slices = 1;
  if (bf16_path && rows * 8 <= NUM_CUS) {
    halves = 1;
    slices = COMBINE_SLICES;
    wpr = 1;
    while (wpr < 16 && 4 * COMBINE_BATCH_SLICE * wpr < seq_splits) wpr *= 2;
  }
  const int64_t cblocks = slices > 1 ? rows * slices : ceil_div64(rows, (wpr < 4 ? 4 : wpr) / wpr) * halves;
  if (blocks > INT32_MAX || cblocks > INT32_MAX || max_splits > INT32_MAX || chunk > INT32_MAX)
    return VERIFY_ATTN_ERR_BAD_DIM;
  pl->M = (int)M;
  pl->nxcd = dv.xcds;
  pl->rows_per_tile = rows_per_tile;
  pl->nk = nk;
  pl->row_tiles = (int)row_tiles;
  pl->chunk = (int)chunk;
  pl->max_splits = (int)max_splits;
  pl->partial_blocks = (int)blocks;
  pl->combine_wpr = wpr;
  pl->combine_halves = halves;
  pl->combine_slices = slices;
  pl->combine_blocks = (int)cblocks;
  // V averages: bf16 on the bf16 path, fp32 on the fp32-input path
  pl->part_o_bytes = (size_t)max_splits * (size_t)M * V_DIM * (bf16_path ? 2 : 4);
  pl->ws_bytes = pl->part_o_bytes + (size_t)max_splits * (size_t)M * 2 * sizeof(float);
  return VERIFY_ATTN_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// The device must be gfx950; checked once per device id (thread-safe: the
// cached answer only ever goes from "unknown" to a fixed value).
int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VERIFY_ATTN_ERR_DEVICE;
  static int cache[64];  // 0 unknown, 1 ok, 2 bad
  if (dev >= 0 && dev < 64) {
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
    if (c) return c == 1 ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VERIFY_ATTN_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) __atomic_store_n(&cache[dev], ok ? 1 : 2, __ATOMIC_RELEASE);
  return ok ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_DEVICE;
}

int launch_partial(const verify_attn_params* p, const Plan& pl, const void* q, const void* kv_pool,
                   const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                   void* workspace, hipStream_t stream) {
  PartialArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv_pool);
  a.slot_idx = slot_idx;
  a.seq_lens = seq_lens;
  a.tree_parent = tree_parent;
  a.part_o = static_cast<uint16_t*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_o_bytes);
  a.B = p->num_seqs;
  a.H = p->num_heads;
  a.T = p->tree_size;
  a.M = pl.M;
  a.row_tiles = pl.row_tiles;
  a.chunk = pl.chunk;
  a.max_splits = pl.max_splits;
  a.max_seq_len = p->max_seq_len;
  a.nxcd = pl.nxcd;
  a.rows_per_tile = pl.rows_per_tile;
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  a.qk_scale_log2 = p->sm_scale * 1.4426950408889634f;
  if (pl.rows_per_tile <= SM_ROWS / 2)
    hipLaunchKernelGGL(verify_attn_partial_small_kernel<1>, dim3(pl.partial_blocks), dim3(NWAVES * 64), 0, stream, a);
  else if (pl.rows_per_tile <= SM_ROWS)
    hipLaunchKernelGGL(verify_attn_partial_small_kernel<2>, dim3(pl.partial_blocks), dim3(NWAVES * 64), 0, stream, a);
  else {
    // some row tile holds at most 96 rows: a wave may have none
    const int last = pl.M - (pl.row_tiles - 1) * ROWS_PER_TILE;
    const bool idle = last <= ROWS_PER_TILE - ROWS_PER_WAVE;
    const dim3 grid(pl.partial_blocks), block(NWAVES * 64);
    if (p->num_seqs == 1 && idle) hipLaunchKernelGGL((verify_attn_partial_kernel<true, true>), grid, block, 0, stream, a);
    else if (p->num_seqs == 1) hipLaunchKernelGGL((verify_attn_partial_kernel<true, false>), grid, block, 0, stream, a);
    else if (idle) hipLaunchKernelGGL((verify_attn_partial_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_attn_partial_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int launch_combine(const verify_attn_params* p, const Plan& pl, const int32_t* seq_lens, void* out,
                   void* workspace, hipStream_t stream, bool f32_out = false) {
  CombineArgs a;
  a.part_o = workspace;
  a.part_ml = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + pl.part_o_bytes);
  a.seq_lens = seq_lens;
  a.out = f32_out ? nullptr : static_cast<uint16_t*>(out);
  a.out_f32 = f32_out ? static_cast<float*>(out) : nullptr;
  a.B = p->num_seqs;
  a.T = p->tree_size;
  a.M = pl.M;
  a.chunk = pl.chunk;
  a.max_splits = pl.max_splits;
  a.max_seq_len = p->max_seq_len;
  const dim3 grid(pl.combine_blocks);
#define VA_COMBINE(W, F) hipLaunchKernelGGL((verify_attn_combine_kernel<W, F>), grid, dim3((W < 4 ? 4 : W) * 64), 0, stream, a)
  if (f32_out) {
    if (pl.combine_halves == 2) hipLaunchKernelGGL((verify_attn_combine_kernel<16, true, true>), grid, dim3(16 * 64), 0, stream, a);
    else switch (pl.combine_wpr) {
      case 16: VA_COMBINE(16, true); break;
      case 8: VA_COMBINE(8, true); break;
      case 4: VA_COMBINE(4, true); break;
      case 2: VA_COMBINE(2, true); break;
      default: VA_COMBINE(1, true); break;
    }
  } else {
    if (pl.combine_slices > 1) {
#define VA_SLICE(W) hipLaunchKernelGGL((verify_attn_combine_slice_kernel<W>), grid, dim3(W * 64), 0, stream, a)
      switch (pl.combine_wpr) {
        case 16: VA_SLICE(16); break;
        case 8: VA_SLICE(8); break;
        case 4: VA_SLICE(4); break;
        case 2: VA_SLICE(2); break;
        default: VA_SLICE(1); break;
      }
#undef VA_SLICE
    } else if (pl.combine_halves == 2) hipLaunchKernelGGL((verify_attn_combine_kernel<16, false, true>), grid, dim3(16 * 64), 0, stream, a);
    else switch (pl.combine_wpr) {
      case 16: VA_COMBINE(16, false); break;
      case 8: VA_COMBINE(8, false); break;
      case 4: VA_COMBINE(4, false); break;
      case 2: VA_COMBINE(2, false); break;
      default: VA_COMBINE(1, false); break;
    }
  }
#undef VA_COMBINE
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int launch_partial_f32(const verify_attn_params* p, const Plan& pl, const float* q, const float* kv_pool,
                       const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                       void* workspace, hipStream_t stream) {
  PartialF32Args a;
  a.q = q;
  a.kv = kv_pool;
  a.slot_idx = slot_idx;
  a.seq_lens = seq_lens;
  a.tree_parent = tree_parent;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_o_bytes);
  a.B = p->num_seqs;
  a.H = p->num_heads;
  a.T = p->tree_size;
  a.M = pl.M;
  a.row_tiles = pl.row_tiles;
  a.chunk = pl.chunk;
  a.max_splits = pl.max_splits;
  a.max_seq_len = p->max_seq_len;
  a.nxcd = pl.nxcd;
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  a.qk_scale_log2 = p->sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(verify_attn_f32_partial_kernel, dim3(pl.partial_blocks), dim3(NWAVES * 64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int check_partial_args(const verify_attn_params* p, Plan* pl, const void* q, const void* kv_pool,
                       const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                       void* workspace, size_t workspace_bytes) {
  const int rc = make_plan(p, pl, current_shape());
  if (rc) return rc;
  if (!q || !kv_pool || !slot_idx || !seq_lens || !tree_parent || !workspace) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(workspace)) return VERIFY_ATTN_ERR_MISALIGNED;
  if (((uintptr_t)slot_idx & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)tree_parent & 3u))
    return VERIFY_ATTN_ERR_MISALIGNED;
  if (workspace_bytes < pl->ws_bytes) return VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL;
  return VERIFY_ATTN_OK;
}

int check_combine_args(const verify_attn_params* p, Plan* pl, const int32_t* seq_lens, void* out,
                       void* workspace, size_t workspace_bytes) {
  const int rc = make_plan(p, pl, current_shape());
  if (rc) return rc;
  if (!seq_lens || !out || !workspace) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(out) || !aligned16(workspace) || ((uintptr_t)seq_lens & 3u)) return VERIFY_ATTN_ERR_MISALIGNED;
  if (workspace_bytes < pl->ws_bytes) return VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL;
  return VERIFY_ATTN_OK;
}

// Split-K partials of verify_attn_noalloc: a file-scope device array instead
// of a caller's workspace, for callers that cannot allocate device memory.
// Each device holds its own copy from the library's load until the process
// ends. Host code never passes `scratch` itself to a kernel (in host code the
// name is a host-side stand-in, not a device address): it passes the device
// address read once per device by scratch_ptr().
static __device__ __align__(256) unsigned char scratch[VERIFY_ATTN_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, read with that device
// current at the first call on it and kept per device id (thread-safe: the
// stored address only ever goes from null to the device's fixed address).
// Returns a status code.
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return VERIFY_ATTN_ERR_DEVICE;
  static void* cache[64];
  void* ptr = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return VERIFY_ATTN_ERR_DEVICE;
    __atomic_store_n(&cache[dev], ptr, __ATOMIC_RELEASE);
  }
  *out = ptr;
  return VERIFY_ATTN_OK;
}

}  // namespace

extern "C" {

size_t verify_attn_workspace_size(const verify_attn_params* p) {
  Plan pl;
  return make_plan(p, &pl, current_shape()) == VERIFY_ATTN_OK ? pl.ws_bytes : 0;
}

int verify_attn_plan_for(const verify_attn_params* p, int32_t fp32_inputs, int32_t num_cus, int32_t num_xcds,
                         verify_attn_plan_info* info) {
  if (!info) return VERIFY_ATTN_ERR_NULL_PTR;
  DevShape dv = current_shape();
  if (num_cus != 0 || num_xcds != 0) dv = DevShape{num_cus, num_xcds};
  Plan pl;
  const int rc = fp32_inputs ? make_plan(p, &pl, dv, F_ROWS_PER_TILE, F_NK) : make_plan(p, &pl, dv);
  if (rc) return rc;
  info->rows_per_tile = pl.rows_per_tile;
  info->row_tiles = pl.row_tiles;
  info->keys_per_split = pl.chunk;
  info->max_splits = pl.max_splits;
  info->partial_blocks = pl.partial_blocks;
  info->combine_blocks = pl.combine_blocks;
  info->threads_per_block = NWAVES * 64;
  info->keys_per_tile = pl.nk;
  return VERIFY_ATTN_OK;
}

int verify_attn_plan(const verify_attn_params* p, verify_attn_plan_info* info) {
  return verify_attn_plan_for(p, 0, 0, 0, info);
}

int verify_attn_partial(const verify_attn_params* p, const void* q, const void* kv_pool,
                        const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = check_partial_args(p, &pl, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace, workspace_bytes);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return launch_partial(p, pl, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace,
                        static_cast<hipStream_t>(stream));
}

int verify_attn_combine(const verify_attn_params* p, const int32_t* seq_lens, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = check_combine_args(p, &pl, seq_lens, out, workspace, workspace_bytes);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return launch_combine(p, pl, seq_lens, out, workspace, static_cast<hipStream_t>(stream));
}

int verify_attn(const verify_attn_params* p, const void* q, const void* kv_pool, const int32_t* slot_idx,
                const int32_t* seq_lens, const int32_t* tree_parent, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = check_partial_args(p, &pl, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace, workspace_bytes);
  if (rc) return rc;
  if (!out) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(out)) return VERIFY_ATTN_ERR_MISALIGNED;
  if ((rc = check_device())) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = launch_partial(p, pl, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace, s))) return rc;
  return launch_combine(p, pl, seq_lens, out, workspace, s);
}

int verify_attn_noalloc(const verify_attn_params* p, const void* q, const void* kv_pool, const int32_t* slot_idx,
                        const int32_t* seq_lens, const int32_t* tree_parent, void* out, void* stream) {
  Plan pl;
  int rc = make_plan(p, &pl, current_shape());
  if (rc) return rc;
  if (!q || !kv_pool || !slot_idx || !seq_lens || !tree_parent || !out) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out)) return VERIFY_ATTN_ERR_MISALIGNED;
  if (((uintptr_t)slot_idx & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)tree_parent & 3u))
    return VERIFY_ATTN_ERR_MISALIGNED;
  if (pl.ws_bytes > VERIFY_ATTN_NOALLOC_SCRATCH_BYTES) return VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = launch_partial(p, pl, q, kv_pool, slot_idx, seq_lens, tree_parent, ws, s))) return rc;
  return launch_combine(p, pl, seq_lens, out, ws, s);
}

size_t verify_attn_f32_workspace_size(const verify_attn_params* p) {
  Plan pl;
  return make_plan(p, &pl, current_shape(), F_ROWS_PER_TILE, F_NK) == VERIFY_ATTN_OK ? pl.ws_bytes : 0;
}

int verify_attn_f32(const verify_attn_params* p, const float* q, const float* kv_pool, const int32_t* slot_idx,
                    const int32_t* seq_lens, const int32_t* tree_parent, float* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(p, &pl, current_shape(), F_ROWS_PER_TILE, F_NK);
  if (rc) return rc;
  if (!q || !kv_pool || !slot_idx || !seq_lens || !tree_parent || !out || !workspace) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || !aligned16(workspace)) return VERIFY_ATTN_ERR_MISALIGNED;
  if (((uintptr_t)slot_idx & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)tree_parent & 3u))
    return VERIFY_ATTN_ERR_MISALIGNED;
  if (workspace_bytes < pl.ws_bytes) return VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if ((rc = check_device())) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = launch_partial_f32(p, pl, q, kv_pool, slot_idx, seq_lens, tree_parent, workspace, s))) return rc;
  return launch_combine(p, pl, seq_lens, out, workspace, s, true);
}

int verify_attn_append_kv(const verify_attn_params* p, const void* kv_new, const int32_t* slot_idx,
                          const int32_t* seq_lens, void* kv_pool, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!kv_new || !slot_idx || !seq_lens || !kv_pool) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(kv_new) || !aligned16(kv_pool)) return VERIFY_ATTN_ERR_MISALIGNED;
  if ((rc = check_device())) return rc;
  AppendArgs a;
  a.kv_new = static_cast<const uint16_t*>(kv_new);
  a.slot_idx = slot_idx;
  a.seq_lens = seq_lens;
  a.kv_pool = static_cast<uint16_t*>(kv_pool);
  a.B = p->num_seqs;
  a.T = p->tree_size;
  a.max_seq_len = p->max_seq_len;
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  const int64_t rows = (int64_t)a.B * a.T;
  if (ceil_div64(rows, 4) > INT32_MAX) return VERIFY_ATTN_ERR_BAD_DIM;
  hipLaunchKernelGGL(verify_attn_append_kernel, dim3((unsigned)ceil_div64(rows, 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int verify_attn_compact_kv(const verify_attn_params* p, const void* kv_pool, const int32_t* slot_idx,
                           void* kv_dst, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!kv_pool || !slot_idx || !kv_dst) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(kv_pool) || !aligned16(kv_dst)) return VERIFY_ATTN_ERR_MISALIGNED;
  if ((rc = check_device())) return rc;
  CompactArgs a;
  a.kv_pool = static_cast<const uint16_t*>(kv_pool);
  a.slot_idx = slot_idx;
  a.kv_dst = static_cast<uint16_t*>(kv_dst);
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  if (ceil_div64(a.total_kv, 4) > INT32_MAX) return VERIFY_ATTN_ERR_BAD_DIM;
  hipLaunchKernelGGL(verify_attn_compact_kernel, dim3((unsigned)ceil_div64(a.total_kv, 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int verify_attn_debug_validate(const verify_attn_params* p, const int32_t* slot_idx, const int32_t* seq_lens,
                               const int32_t* tree_parent, int32_t* flags, void* stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (!slot_idx || !seq_lens || !tree_parent || !flags) return VERIFY_ATTN_ERR_NULL_PTR;
  if (((uintptr_t)slot_idx & 3u) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)tree_parent & 3u) ||
      ((uintptr_t)flags & 3u))
    return VERIFY_ATTN_ERR_MISALIGNED;
  if ((rc = check_device())) return rc;
  ValidateArgs a;
  a.slot_idx = slot_idx;
  a.seq_lens = seq_lens;
  a.tree_parent = tree_parent;
  a.flags = flags;
  a.B = p->num_seqs;
  a.T = p->tree_size;
  a.max_seq_len = p->max_seq_len;
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(verify_attn_validate_clear, dim3(1), dim3(64), 0, s, flags);
  const int64_t blocks = std::min<int64_t>(1024, ceil_div64(std::max<int64_t>(a.total_kv, (int64_t)a.B * a.T), 256));
  hipLaunchKernelGGL(verify_attn_validate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

const char* verify_attn_strerror(int status) {
  switch (status) {
    case VERIFY_ATTN_OK: return "ok";
    case VERIFY_ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case VERIFY_ATTN_ERR_BAD_DIM: return "invalid dimension (num_seqs, num_heads, kv_dim=576, v_dim=512, "
                                         "page_size, pool_slots, sm_scale or reserved)";
    case VERIFY_ATTN_ERR_TREE_TOO_LARGE: return "tree_size must be in 1..64";
    case VERIFY_ATTN_ERR_MISALIGNED: return "q, kv_pool, out and workspace must be 16-byte aligned";
    case VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than verify_attn_workspace_size()";
    case VERIFY_ATTN_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case VERIFY_ATTN_ERR_BAD_SEQ: return "inconsistent sequence sizes (max_seq_len, total_kv)";
    case VERIFY_ATTN_ERR_BAD_SPLIT: return "nsplit must be >= 0";
    case VERIFY_ATTN_ERR_DEVICE: return "no gfx950 device is current";
    case VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more split-K scratch than verify_attn_noalloc holds "
             "(VERIFY_ATTN_NOALLOC_SCRATCH_BYTES = 80 MiB); use verify_attn with a workspace";
    default: return "unknown status";
  }
}

int verify_attn_version(void) { return VERIFY_ATTN_VERSION; }

}  // extern "C"
