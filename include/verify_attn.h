/*
 * verify_attn.h — C ABI of the MI355X (gfx950) MLA tree-verify attention library.
 *
 * The operation: speculative-decoding verify attention for Multi-head Latent
 * Attention. The draft tokens of a DDTree draft tree are verified against the
 * full latent KV cache ("The Milestone Commit", Input Knowledge). The call
 * takes the serving engine's extend layout: per sequence, the prefix's KV slot
 * list followed by the draft tokens' slots, with the draft-token mask built
 * over prefix + q_len positions ("The Checkpoint Report", Mistakes and
 * Incorrect Assumptions). Here the mask is not passed in; it is derived on the
 * device from each node's parent pointer (a node sees the whole prefix, itself
 * and its tree ancestors).
 *
 * For sequence b, draft node t and head h (row r = t*H + h of the sequence):
 *   P_b      = seq_lens[b] - T
 *   K_j      = kv_pool[slot_idx[seg_b + j]]   (576 values: 512 latent + 64 rope)
 *   V_j      = K_j[0:512]
 *   visible  = every prefix key j < P_b, and the tree key P_b + u when u is t
 *              or an ancestor of t
 *   out[b,t,h,:] = softmax_j(sm_scale * q[b,t,h,:] . K_j) weighted sum of V_j
 *
 * The library is the paged, bf16, multi-sequence variant behind a C ABI
 * ("The Checkpoint Report", Architecture of the Report) and capture-safe: it consumes the
 * caller's buffers, takes a caller-allocated workspace, makes no host
 * synchronisation and no device allocation inside the call ("The Commit That
 * Locked In 6x Decode", 1. Capture-Safe Design), so a call can be recorded in a
 * HIP graph and replayed. The work is split over the KV sequence (split-K) and
 * the per-split softmax partials are merged by a log-sum-exp combine ("The
 * Milestone Commit", Thinking Process; "The Commit That Locked In 6x Decode",
 * 2. NSPLIT=64 for TP8 Occupancy).
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously and the call returns without waiting.
 *  - Status: 0 on success, a negative VERIFY_ATTN_ERR_* code otherwise. On an
 *    error nothing is enqueued. No entry point prints, aborts or throws.
 *  - Host-known parameters (the params struct) are validated on the host.
 *    Device-resident contents (slot_idx, seq_lens, tree_parent) cannot be
 *    checked without a host synchronisation; their validity is a
 *    precondition. The kernels clamp every index they derive from them, so
 *    invalid contents give meaningless output but never an out-of-bounds
 *    access or a hang.
 *  - The library holds no mutable global state; calls on different streams
 *    with different workspaces may run concurrently.
 */
#ifndef MLA_TREE_VERIFY_ATTN_H
#define MLA_TREE_VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VERIFY_ATTN_KV_DIM 576   /* latent (512) + rope (64) bf16 values per KV row */
#define VERIFY_ATTN_V_DIM 512    /* V is the first 512 values of the same row */
#define VERIFY_ATTN_MAX_TREE 64  /* tree nodes per sequence (64-bit ancestor masks) */

enum verify_attn_status {
  VERIFY_ATTN_OK = 0,
  VERIFY_ATTN_ERR_NULL_PTR = -1,            /* a required pointer is NULL */
  VERIFY_ATTN_ERR_BAD_DIM = -2,             /* B/H < 1, kv_dim != 576, v_dim != 512, H*T > 2^20,
                                               a grid, split count or split length past 2^31 - 1, ... */
  VERIFY_ATTN_ERR_TREE_TOO_LARGE = -3,      /* tree_size outside 1..64 */
  VERIFY_ATTN_ERR_MISALIGNED = -4,          /* q/kv_pool/out/workspace not 16-byte aligned */
  VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL = -5, /* workspace_bytes < verify_attn_workspace_size() */
  VERIFY_ATTN_ERR_LAUNCH_FAILED = -6,       /* the HIP runtime rejected a kernel launch */
  VERIFY_ATTN_ERR_BAD_SEQ = -7,             /* max_seq_len < tree_size, total_kv < B*T, ... */
  VERIFY_ATTN_ERR_BAD_SPLIT = -8,           /* nsplit < 0 */
  VERIFY_ATTN_ERR_DEVICE = -9,              /* no device, or the device is not gfx950 */
  VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL = -10   /* verify_attn_noalloc: partials exceed its scratch */
};

/*
 * Host-known shape of one call. Everything here is fixed when a call is
 * recorded into a HIP graph; the device buffers' contents may change between
 * replays.
 */
typedef struct verify_attn_params {
  int32_t num_seqs;    /* B >= 1 sequences in the batch */
  int32_t num_heads;   /* H >= 1 query heads (all share the one latent KV row) */
  int32_t tree_size;   /* T in 1..64 draft-tree nodes per sequence (same T for all) */
  int32_t kv_dim;      /* must be 576 */
  int32_t v_dim;       /* must be 512 */
  int32_t page_size;   /* >= 1; layout hint only (slot_idx is per token either way) */
  int32_t max_seq_len; /* >= every seq_lens[b] and >= T; sizes the launch, no device read */
  int32_t nsplit;      /* 0 = automatic; else the maximum number of KV splits of one sequence */
  int64_t total_kv;    /* number of entries of slot_idx (= sum of seq_lens), >= B*T */
  int64_t pool_slots;  /* number of rows of kv_pool, >= 1 */
  float sm_scale;      /* softmax scale applied to q . K (e.g. 1/sqrt(192)) */
  int32_t reserved;    /* must be 0 */
} verify_attn_params;

/*
 * Bytes of device workspace one call needs for these params (split-K
 * partials), or 0 when the params are invalid. The workspace is scratch: its
 * contents need no initialisation and are meaningless after the call. Calls
 * that may run concurrently need distinct workspaces.
 */
size_t verify_attn_workspace_size(const verify_attn_params* p);

/*
 * The verify attention (partial kernel, then combine kernel, on `stream`).
 *   q           bf16 [B, T, H, 576], contiguous, 16-byte aligned
 *   kv_pool     bf16 [pool_slots, 576], contiguous, 16-byte aligned
 *   slot_idx    int32 [total_kv]: per sequence (in order), seq_lens[b] - T prefix
 *               slots then the T tree nodes' own slots in node order
 *   seq_lens    int32 [B]: P_b + T, each in [T, max_seq_len]
 *   tree_parent int32 [B, T]: parent node of node t in [-1, t-1]; -1 = the node
 *               hangs directly off the prefix
 *   out         bf16 [B, T, H, 512], contiguous, 16-byte aligned (written, RNE)
 *   workspace   >= verify_attn_workspace_size(p) bytes, 16-byte aligned
 */
int verify_attn(const verify_attn_params* p, const void* q, const void* kv_pool,
                const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * verify_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation). The split-K partials
 * go to a scratch array inside the library instead: VERIFY_ATTN_NOALLOC_SCRATCH_BYTES
 * of device memory per GPU, reserved when the library's code is loaded on that
 * GPU and held until the process ends. Same arguments, layouts and result as
 * verify_attn (the same plan and kernels, so the same bits). Makes no
 * allocation and no host synchronisation; the scratch address is looked up
 * once per device, at the first call on it.
 *   Limit: calls whose verify_attn_workspace_size(p) exceeds the scratch
 *   return VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL and enqueue nothing. One split
 *   round over the device's compute units fits (e.g. H=8, T=64 or H=64, T=64
 *   at 65k tokens: 32.25 MiB); ragged batches needing several rounds may not.
 *   Sharing: every call on a GPU uses that GPU's one scratch array, which
 *   keeps the last call's contents (nothing in it needs clearing: each call
 *   writes every partial it reads). Calls that may overlap on one GPU (other
 *   streams, other threads) race on it and give wrong results; order them on
 *   one stream, or use verify_attn with distinct workspaces.
 */
#define VERIFY_ATTN_NOALLOC_SCRATCH_BYTES (80u << 20)
int verify_attn_noalloc(const verify_attn_params* p, const void* q, const void* kv_pool,
                        const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* tree_parent,
                        void* out, void* stream);

/*
 * The two stages of verify_attn, separately (same arguments and checks).
 * verify_attn_partial writes the per-split softmax partials (running max and
 * running sum in fp32; the split's V average, its weighted V sum divided by the
 * running sum, rounded to bf16, nearest even) into the workspace;
 * verify_attn_combine reads them and writes `out`.
 * verify_attn == partial followed by combine. Exposed so a profiler or
 * benchmark can time the stages on their own.
 */
int verify_attn_partial(const verify_attn_params* p, const void* q, const void* kv_pool,
                        const int32_t* slot_idx, const int32_t* seq_lens,
                        const int32_t* tree_parent, void* workspace, size_t workspace_bytes,
                        void* stream);
int verify_attn_combine(const verify_attn_params* p, const int32_t* seq_lens, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The launch decomposition chosen for these params (informational; the same
 * values the calls use). The work is split over the KV positions of each
 * sequence; a split's keys are processed in tiles of keys_per_tile, with one
 * running softmax maximum per query row and split. Returns a status code.
 *
 * The decomposition depends on the device: its compute units (one partial
 * workgroup each per round) and its XCDs (workgroups are dealt to them
 * round-robin). verify_attn_plan, verify_attn_workspace_size and the calls
 * plan for the current device (read once per device: multiProcessorCount,
 * which is smaller under a CU-partitioned mode, and the XCD count); without a
 * current device, for a whole MI355X (256 compute units in 8 XCDs).
 */
typedef struct verify_attn_plan_info {
  int32_t rows_per_tile;   /* query rows (of H*T) per workgroup */
  int32_t row_tiles;       /* ceil(H*T / rows_per_tile) */
  int32_t keys_per_split;  /* KV positions per split */
  int32_t max_splits;      /* upper bound on the total number of splits over all sequences */
  int32_t partial_blocks;  /* workgroups of the partial kernel */
  int32_t combine_blocks;  /* workgroups of the combine kernel */
  int32_t threads_per_block;
  int32_t keys_per_tile;   /* KV positions per tile of the partial kernel */
} verify_attn_plan_info;

int verify_attn_plan(const verify_attn_params* p, verify_attn_plan_info* info);

/*
 * The same for either input type (fp32_inputs != 0: verify_attn_f32) and an
 * explicit device shape: num_cus compute units in num_xcds XCDs (1 <= num_xcds
 * <= num_cus <= 65536), or the current device's when both are 0. Host only:
 * touches no device memory. Returns a status code (VERIFY_ATTN_ERR_BAD_DIM
 * for an invalid shape).
 */
int verify_attn_plan_for(const verify_attn_params* p, int32_t fp32_inputs, int32_t num_cus, int32_t num_xcds,
                         verify_attn_plan_info* info);

/*
 * Draft-row KV append: the step right before verify in the extend layout,
 * where the draft tokens' own KV slots follow each sequence's prefix slots
 * ("The Checkpoint Report", Mistakes and Incorrect Assumptions). Row (b, t) of
 * kv_new (the latent row of draft-tree node t of sequence b) is copied to
 *   kv_pool[slot_idx[seg_b + seq_lens[b] - T + t]],   seg_b = sum_{b' < b} seq_lens[b'],
 * so that a following verify_attn on the same stream sees the tree nodes' rows.
 * Uses num_seqs, tree_size, max_seq_len, total_kv and pool_slots of `p` (the
 * params of the verify call it precedes; the same validation applies).
 *   kv_new   bf16 [B, T, 576], contiguous, 16-byte aligned (read)
 *   slot_idx, seq_lens as for verify_attn (read)
 *   kv_pool  bf16 [pool_slots, 576], 16-byte aligned; the B*T target rows are written
 * Enqueued on `stream`; no allocation and no host synchronisation, so it can be
 * recorded in the same HIP graph as the verify call. Slots outside
 * [0, pool_slots) are skipped; if two nodes share a slot, which row lands is
 * unspecified. Status codes as above.
 */
int verify_attn_append_kv(const verify_attn_params* p, const void* kv_new, const int32_t* slot_idx,
                          const int32_t* seq_lens, void* kv_pool, void* stream);

/*
 * fp32-input variant ("The Checkpoint Report", Architecture of the Report: the
 * first kernel of the pages took fp32 data with 16-byte vector loads): the same
 * operation as verify_attn on binary32 q and KV rows, computed in fp32
 * throughout (MFMA 16x16x4 f32; the softmax weights stay fp32), fp32 output.
 *   q        float [B, T, H, 576], 16-byte aligned
 *   kv_pool  float [pool_slots, 576] (2,304-byte rows), 16-byte aligned
 *   out      float [B, T, H, 512], 16-byte aligned
 *   slot_idx, seq_lens, tree_parent, p: as for verify_attn.
 *   workspace: at least verify_attn_f32_workspace_size(p) bytes, 16-byte
 *   aligned (caller-owned; its own size, not verify_attn_workspace_size).
 * Two kernels on `stream`; no allocation, no host synchronisation (graph
 * capturable). Status codes as for verify_attn.
 */
size_t verify_attn_f32_workspace_size(const verify_attn_params* p);
int verify_attn_f32(const verify_attn_params* p, const float* q, const float* kv_pool, const int32_t* slot_idx,
                    const int32_t* seq_lens, const int32_t* tree_parent, float* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * KV defragmentation: copy every referenced latent row into consecutive rows,
 *   kv_dst[i] = kv_pool[slot_idx[i]]   for i < total_kv,
 * i.e. each sequence's KV (prefix rows, then its tree nodes' rows) becomes one
 * contiguous run of rows, as the pages' planned defragmentation phase keeps a
 * request's KV contiguous ("The Checkpoint Report", Architecture of the Report and Input
 * Knowledge). A verify_attn call on kv_dst with slot_idx[i] = i (page_size 64)
 * then gives the same result bit for bit. Uses total_kv and pool_slots of `p`.
 *   kv_pool  bf16 [pool_slots, 576], 16-byte aligned (read)
 *   slot_idx int32 [total_kv] (read)
 *   kv_dst   bf16 [total_kv, 576], 16-byte aligned, must not overlap kv_pool (written)
 * Enqueued on `stream`; no allocation, no host synchronisation. A slot outside
 * [0, pool_slots) yields a row of zeros. Status codes as above.
 */
int verify_attn_compact_kv(const verify_attn_params* p, const void* kv_pool, const int32_t* slot_idx,
                           void* kv_dst, void* stream);

/*
 * Debug check of the device-resident inputs that the other entry points take
 * as a precondition (for tests and bring-up, not for the hot path): enqueues
 * a clear of *flags and a scan that sets
 *   VERIFY_ATTN_BAD_LENGTH  some seq_lens[b] outside [tree_size, max_seq_len]
 *   VERIFY_ATTN_BAD_TOTAL   sum of seq_lens > total_kv
 *   VERIFY_ATTN_BAD_PARENT  some tree_parent[b][t] outside [-1, t-1]
 *   VERIFY_ATTN_BAD_SLOT    some slot_idx[i] (i < total_kv) outside [0, pool_slots)
 * flags: one int32 in device memory (caller-owned; read it after the stream
 * has run). No allocation or host synchronisation. Status codes as above.
 */
#define VERIFY_ATTN_BAD_LENGTH 1
#define VERIFY_ATTN_BAD_TOTAL 2
#define VERIFY_ATTN_BAD_PARENT 4
#define VERIFY_ATTN_BAD_SLOT 8
int verify_attn_debug_validate(const verify_attn_params* p, const int32_t* slot_idx, const int32_t* seq_lens,
                               const int32_t* tree_parent, int32_t* flags, void* stream);

/* Static description of a status code (never NULL). */
const char* verify_attn_strerror(int status);

/* ABI version of this header: (major << 16) | minor (minor 1: verify_attn_append_kv; 2: verify_attn_compact_kv;
   3: verify_attn_f32; 4: verify_attn_debug_validate; 5: verify_attn_plan_for, keys_per_tile in
   verify_attn_plan_info, plans for the current device's compute units and XCDs; 6: verify_attn_noalloc). */
int verify_attn_version(void);

#define VERIFY_ATTN_VERSION ((1 << 16) | 6)

#ifdef __cplusplus
}
#endif

#endif /* MLA_TREE_VERIFY_ATTN_H */
