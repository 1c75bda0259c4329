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
//  - one workgroup = 4 waves = 64 query rows (rows are (node, head) pairs of one
//    sequence, r = t*H + h) x one split of the sequence's KV positions;
//  - KV tiles of 32 rows (36 KB) are gathered straight into LDS with 16-byte
//    direct-to-LDS loads, one slot-table lookup per row, double-buffered;
//  - S^T = K Q^T and O^T += V^T P^T on MFMA 16x16x32 bf16, so every lane holds
//    whole query rows of both the scores and the accumulator (the softmax state
//    of a row never leaves its lanes); V^T comes from the K-major LDS tile with
//    the LDS transpose read;
//  - fp32 online softmax in base 2, tree mask from per-node 64-bit ancestor
//    masks built on the device from the parent pointers;
//  - a log-sum-exp combine kernel merges the splits and rounds to bf16.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/verify_attn.h"

namespace {

constexpr int KV_DIM = 576;
constexpr int V_DIM = 512;
constexpr int MAX_TREE = 64;

// Partial kernel geometry.
constexpr int NW = 4;                      // waves per workgroup
constexpr int ROWS_PER_WAVE = 16;          // query rows per wave (MFMA N for QK, N for PV)
constexpr int ROWS_PER_TILE = NW * ROWS_PER_WAVE;  // 64
constexpr int NK = 32;                     // KV rows per LDS tile
constexpr int ROWS_PER_WAVE_LOAD = NK / NW;  // 8 KV rows loaded by each wave
constexpr int CHUNK_GROUPS = KV_DIM / 64;  // 9 groups of 64 bf16 (8 x 16 B) per KV row
constexpr int GROUP_BYTES = NK * 128;      // one group for all NK rows: 4 KB
constexpr int TILE_BYTES = CHUNK_GROUPS * GROUP_BYTES;  // 36 KB
constexpr int QK_STEPS = KV_DIM / 32;      // 18 MFMA k-steps of 32 features
constexpr int PV_BLOCKS = V_DIM / 16;      // 32 output blocks of 16 features
constexpr float LAZY_RESCALE_LOG2 = 8.0f;  // running max is raised only past +8 (base 2)

constexpr int COMBINE_ROWS_PER_BLOCK = 4;  // one wave per output row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

struct Plan {
  int M;               // H*T rows per sequence
  int row_tiles;       // ceil(M / ROWS_PER_TILE)
  int chunk;           // keys per split (multiple of NK)
  int max_splits;      // bound on the total number of splits
  int partial_blocks;  // multiple of 8
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
  float* part_o;   // [max_splits][M][512]
  float* part_ml;  // [max_splits][M][2] = (running max (base 2, scaled), running sum)
  int B, H, T, M;
  int row_tiles, chunk, max_splits, max_seq_len;
  int64_t total_kv, pool_slots;
  float qk_scale_log2;  // sm_scale * log2(e)
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* seq_lens;
  uint16_t* out;
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

// Swizzle of the 16-byte chunk position inside a 128-byte row segment, so that
// the MFMA operand reads (8 consecutive KV rows, same column) and the
// transpose reads (4 rows x 2 chunks) hit distinct LDS bank groups.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

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
#pragma clang diagnostic pop

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------ partial kernel
//
// LDS tile layout (36 KB per buffer, two buffers): KV row k (0..31) of the
// tile, 16-byte chunk c (0..71) of that row lives at
//   (c / 8) * 4096 + k * 128 + ((c % 8) ^ swz(k)) * 16.
// Wave w loads KV rows 8w..8w+7 of each tile: 9 direct-to-LDS loads of 1 KB
// (one per chunk group), lane -> (row 8w + lane/8, chunk position lane%8).
//
// Per wave, per tile (16 query rows, 32 keys):
//   S^T[32 keys x 16 rows] = K[32 x 576] . Q^T   : 2 key blocks x 18 MFMA 16x16x32
//   lane l holds keys {4g+i, 16+4g+i} (g = l/16, i < 4) of query row l%16
//   P^T (bf16) is then exactly the B operand of O^T += V^T P^T (k = 32 keys),
//   and V^T is read with ds_read_tr16_b64 from the same K-major tile.
//   O^T lane l holds features {16cb + 4g + i} of query row l%16.
__global__ __launch_bounds__(NW * 64, 2) void verify_attn_partial_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE_BYTES];
  __shared__ unsigned long long anc_s[MAX_TREE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so hand
  // each XCD a contiguous range of (split, row tile) pairs; the row tiles of
  // one split then share that XCD's L2 for their KV reads.
  const int per_xcd = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int g = logical / a.row_tiles;
  const int rt = logical - g * a.row_tiles;
  if (g >= a.max_splits) return;

  SplitLoc loc;
  if (!locate_split(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, g, false, &loc)) return;
  loc.b = __builtin_amdgcn_readfirstlane(loc.b);
  loc.g0 = __builtin_amdgcn_readfirstlane(loc.g0);
  loc.len = __builtin_amdgcn_readfirstlane(loc.len);
  loc.seg = ((int64_t)__builtin_amdgcn_readfirstlane((int)(loc.seg >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)loc.seg);
  const int split = g - loc.g0;
  const int k0 = split * a.chunk;
  const int k1 = min(k0 + a.chunk, loc.len);
  const int P = loc.len - a.T;

  // Ancestor masks of this sequence's tree (bit u of anc[t]: node u is t or an
  // ancestor of t). Parent pointers outside [-1, u-1] end the walk.
  if (threadIdx.x < a.T) {
    const int32_t* par = a.tree_parent + (int64_t)loc.b * a.T;
    unsigned long long m = 0;
    int u = threadIdx.x;
    for (int step = 0; step < a.T && u >= 0; ++step) {
      m |= 1ull << u;
      const int p = par[u];
      u = (p < u) ? p : -1;
    }
    anc_s[threadIdx.x] = m;
  }

  // Query fragments (B operand of S^T = K Q^T): 8 features per k-step.
  const int qrow = rt * ROWS_PER_TILE + wave * ROWS_PER_WAVE + (lane & 15);
  const bool row_ok = qrow < a.M;
  const int lg = lane >> 4;  // lane group 0..3
  bf16x8 qf[QK_STEPS];
  {
    const uint16_t* src = a.q + ((int64_t)loc.b * a.M + (row_ok ? qrow : 0)) * KV_DIM + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(src + 32 * ks);
      if (!row_ok) v = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Loader lane mapping.
  const int ld_row = wave * ROWS_PER_WAVE_LOAD + (lane >> 3);
  const int ld_pos = lane & 7;
  const int ld_elem = 8 * (ld_pos ^ swz(ld_row));
  const int64_t slot_hi = a.total_kv - 1;
  const int64_t pool_hi = a.pool_slots - 1;
  // The slot-table value is clamped where it is used, so that the load's
  // latency overlaps the previous tile's compute.
  auto load_slot = [&](int key0) -> int {
    int key = key0 + ld_row;
    key = key < k1 ? key : k1 - 1;
    int64_t si = loc.seg + key;
    si = si < slot_hi ? si : slot_hi;
    return a.slot_idx[si];
  };
  const uint32_t smem_base = lds_addr(smem);
  auto issue_tile = [&](int slot, uint32_t buf) {
    int64_t s = slot < 0 ? 0 : slot;
    s = s > pool_hi ? pool_hi : s;
    const uint16_t* src = a.kv + s * KV_DIM + ld_elem;
    const uint32_t dst = buf + wave * (ROWS_PER_WAVE_LOAD * 128);
#pragma unroll
    for (int j = 0; j < CHUNK_GROUPS; ++j) load_to_lds16(src + 64 * j, dst + j * GROUP_BYTES);
  };

  // Operand read offsets inside a tile.
  const int ql = lane & 15;
  int qk_off[2][2];  // [k-step parity][key block]
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kr = 16 * kb + ql;
      qk_off[par][kb] = kr * 128 + ((((4 * par + lg)) ^ swz(kr)) << 4);
    }
  int pv_off[4][2];  // [cb % 4][key half]
  {
    const int r = ql >> 2, c = ql & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int kr = 16 * hf + 4 * lg + r;
        pv_off[j][hf] = kr * 128 + (((2 * j + (c >> 1)) ^ swz(kr)) << 4) + 8 * (c & 1);
      }
  }

  f32x4 o[PV_BLOCKS];
#pragma unroll
  for (int cb = 0; cb < PV_BLOCKS; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running reference max (base-2 scaled scores)
  float l_run = 0.f;        // this lane's share of the running sum

  const int ntiles = (k1 - k0 + NK - 1) / NK;
  int slot_next = load_slot(k0);
  issue_tile(slot_next, smem_base);
  if (ntiles > 1) slot_next = load_slot(k0 + NK);

  __syncthreads();  // anc_s visible
  const unsigned long long anc = anc_s[row_ok ? qrow / a.H : 0];

  for (int it = 0; it < ntiles; ++it) {
    const uint32_t cur = smem_base + (it & 1) * TILE_BYTES;
    if (it + 1 < ntiles) {
      issue_tile(slot_next, smem_base + ((it + 1) & 1) * TILE_BYTES);
      if (it + 2 < ntiles) {
        slot_next = load_slot(k0 + (it + 2) * NK);
        wait_vmcnt<CHUNK_GROUPS + 1>();
      } else {
        wait_vmcnt<CHUNK_GROUPS>();
      }
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();

    // ---- S^T = K Q^T
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      const uint32_t base = cur + (ks >> 1) * GROUP_BYTES;
      const bf16x8 k0v = lds_read_b128(base + qk_off[ks & 1][0]);
      const bf16x8 k1v = lds_read_b128(base + qk_off[ks & 1][1]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0v, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1v, qf[ks], s1, 0, 0, 0);
    }

    // ---- scale, tree mask, online softmax (base 2)
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i] * a.qk_scale_log2;
      sv[4 + i] = s1[i] * a.qk_scale_log2;
    }
    const int kt = k0 + it * NK;
    if (kt + NK > k1 || kt + NK > P) {
      const int kb0 = kt + 4 * lg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb0 + (e < 4 ? e : 12 + e);
        const int u = key - P;
        const bool vis = key < k1 && (u < 0 || ((anc >> (u & 63)) & 1ull));
        sv[e] = vis ? sv[e] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool raise = mx > m_run + LAZY_RESCALE_LOG2;
    if (__ballot(raise)) {
      const float alpha = raise ? exp2f(m_run - mx) : 1.0f;  // m_run = -inf -> 0
      m_run = raise ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < PV_BLOCKS; ++cb) o[cb] *= alpha;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = exp2f(sv[e] - mu);
    const bf16x8 pb = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                       (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
    {
      // The running sum uses the same bf16-rounded weights that enter O.
      const u32x4 w = __builtin_bit_cast(u32x4, pb);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += __builtin_bit_cast(float, w[i] << 16) + __builtin_bit_cast(float, w[i] & 0xffff0000u);
      l_run += acc;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int cb = 0; cb < PV_BLOCKS; ++cb) {
      const uint32_t base = cur + (cb >> 2) * GROUP_BYTES;
      const bf16x4 v0 = lds_read_tr(base + pv_off[cb & 3][0]);
      const bf16x4 v1 = lds_read_tr(base + pv_off[cb & 3][1]);
      const bf16x8 vt = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb, o[cb], 0, 0, 0);
    }
    lds_barrier();  // every wave is done with `cur` before it is refilled
  }

  // ---- partial results of this split
  float l_row = l_run + __shfl_xor(l_run, 16);
  l_row += __shfl_xor(l_row, 32);
  if (row_ok) {
    const int64_t rowid = (int64_t)g * a.M + qrow;
    float* po = a.part_o + rowid * V_DIM + 4 * lg;
#pragma unroll
    for (int cb = 0; cb < PV_BLOCKS; ++cb) *reinterpret_cast<f32x4*>(po + 16 * cb) = o[cb];
    if (lg == 0) {
      a.part_ml[2 * rowid] = m_run;
      a.part_ml[2 * rowid + 1] = l_row;
    }
  }
}

// ------------------------------------------------------------ combine kernel
// One wave per output row (b, r); lane covers 8 consecutive features.
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s, in
// split order, rounded to bf16 (nearest even).
__global__ __launch_bounds__(COMBINE_ROWS_PER_BLOCK * 64) void verify_attn_combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * COMBINE_ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (grow >= (int64_t)a.B * a.M) return;
  const int b = (int)(grow / a.M);
  const int row = (int)(grow - (int64_t)b * a.M);

  SplitLoc loc;
  if (!locate_split(a.seq_lens, a.B, a.T, a.max_seq_len, a.chunk, b, true, &loc)) return;
  int g_end = loc.g0 + loc.n_splits;
  g_end = g_end < a.max_splits ? g_end : a.max_splits;

  float mmax = -INFINITY;
  for (int g = loc.g0; g < g_end; ++g) mmax = fmaxf(mmax, a.part_ml[2 * ((int64_t)g * a.M + row)]);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int g = loc.g0; g < g_end; ++g) {
    const int64_t rowid = (int64_t)g * a.M + row;
    const float m = a.part_ml[2 * rowid];
    const float l = a.part_ml[2 * rowid + 1];
    const float w = (m == -INFINITY) ? 0.f : exp2f(m - mmax);
    const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + rowid * V_DIM + 8 * lane);
    acc0 += w * src[0];
    acc1 += w * src[1];
    L += w * l;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  u32x4 packed;
  packed[0] = (uint32_t)f32_to_bf16_rne(acc0[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc0[1] * inv) << 16);
  packed[1] = (uint32_t)f32_to_bf16_rne(acc0[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc0[3] * inv) << 16);
  packed[2] = (uint32_t)f32_to_bf16_rne(acc1[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc1[1] * inv) << 16);
  packed[3] = (uint32_t)f32_to_bf16_rne(acc1[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc1[3] * inv) << 16);
  *reinterpret_cast<u32x4*>(a.out + grow * V_DIM + 8 * lane) = packed;
}

// ------------------------------------------------------------------- host

constexpr int TARGET_BLOCKS = 512;  // partial workgroups the automatic split aims for
constexpr int MIN_CHUNK = 256;      // keys per split below which partials dominate

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

int make_plan(const verify_attn_params* p, Plan* pl) {
  const int rc = validate(p);
  if (rc) return rc;
  const int64_t M = (int64_t)p->num_heads * p->tree_size;
  const int64_t row_tiles = ceil_div64(M, ROWS_PER_TILE);
  int64_t chunk;
  if (p->nsplit > 0) {
    chunk = ceil_div64(p->max_seq_len, p->nsplit);
  } else {
    chunk = ceil_div64(p->total_kv * row_tiles, TARGET_BLOCKS);
    if (chunk < MIN_CHUNK) chunk = MIN_CHUNK;
  }
  chunk = ceil_div64(chunk, NK) * NK;
  const int64_t len_cap = ceil_div64(p->max_seq_len, NK) * NK;
  if (chunk > len_cap) chunk = len_cap;
  const int64_t max_splits = ceil_div64(p->total_kv, chunk) + p->num_seqs;
  const int64_t blocks = ceil_div64(max_splits * row_tiles, 8) * 8;
  const int64_t cblocks = ceil_div64((int64_t)p->num_seqs * M, COMBINE_ROWS_PER_BLOCK);
  if (blocks > INT32_MAX || cblocks > INT32_MAX || max_splits > INT32_MAX) return VERIFY_ATTN_ERR_BAD_DIM;
  pl->M = (int)M;
  pl->row_tiles = (int)row_tiles;
  pl->chunk = (int)chunk;
  pl->max_splits = (int)max_splits;
  pl->partial_blocks = (int)blocks;
  pl->combine_blocks = (int)cblocks;
  pl->part_o_bytes = (size_t)max_splits * (size_t)M * V_DIM * sizeof(float);
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
  a.total_kv = p->total_kv;
  a.pool_slots = p->pool_slots;
  a.qk_scale_log2 = p->sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(verify_attn_partial_kernel, dim3(pl.partial_blocks), dim3(NW * 64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int launch_combine(const verify_attn_params* p, const Plan& pl, const int32_t* seq_lens, void* out,
                   void* workspace, hipStream_t stream) {
  CombineArgs a;
  a.part_o = static_cast<const float*>(workspace);
  a.part_ml = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + pl.part_o_bytes);
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.B = p->num_seqs;
  a.T = p->tree_size;
  a.M = pl.M;
  a.chunk = pl.chunk;
  a.max_splits = pl.max_splits;
  a.max_seq_len = p->max_seq_len;
  hipLaunchKernelGGL(verify_attn_combine_kernel, dim3(pl.combine_blocks), dim3(COMBINE_ROWS_PER_BLOCK * 64),
                     0, stream, a);
  return hipGetLastError() == hipSuccess ? VERIFY_ATTN_OK : VERIFY_ATTN_ERR_LAUNCH_FAILED;
}

int check_partial_args(const verify_attn_params* p, Plan* pl, const void* q, const void* kv_pool,
                       const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                       void* workspace, size_t workspace_bytes) {
  const int rc = make_plan(p, pl);
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
  const int rc = make_plan(p, pl);
  if (rc) return rc;
  if (!seq_lens || !out || !workspace) return VERIFY_ATTN_ERR_NULL_PTR;
  if (!aligned16(out) || !aligned16(workspace) || ((uintptr_t)seq_lens & 3u)) return VERIFY_ATTN_ERR_MISALIGNED;
  if (workspace_bytes < pl->ws_bytes) return VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL;
  return VERIFY_ATTN_OK;
}

}  // namespace

extern "C" {

size_t verify_attn_workspace_size(const verify_attn_params* p) {
  Plan pl;
  return make_plan(p, &pl) == VERIFY_ATTN_OK ? pl.ws_bytes : 0;
}

int verify_attn_plan(const verify_attn_params* p, verify_attn_plan_info* info) {
  if (!info) return VERIFY_ATTN_ERR_NULL_PTR;
  Plan pl;
  const int rc = make_plan(p, &pl);
  if (rc) return rc;
  info->rows_per_tile = ROWS_PER_TILE;
  info->row_tiles = pl.row_tiles;
  info->keys_per_split = pl.chunk;
  info->max_splits = pl.max_splits;
  info->partial_blocks = pl.partial_blocks;
  info->combine_blocks = pl.combine_blocks;
  info->threads_per_block = NW * 64;
  info->reserved = 0;
  return VERIFY_ATTN_OK;
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
    default: return "unknown status";
  }
}

int verify_attn_version(void) { return VERIFY_ATTN_VERSION; }

}  // extern "C"
