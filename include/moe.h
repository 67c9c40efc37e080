/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN layer.
 *
 * The layer: a router picks, per token, the k experts with the largest logits
 * and weights them by the softmax of those k logits; the tokens are grouped by
 * expert; each expert runs a SwiGLU FFN whose weights are stored in a low-bit
 * block format; the expert outputs are summed back in token order with the
 * gate weights.  Sources for what is computed:
 *   - only a few experts per token run (10 of 512 in each of 48 layers of the
 *     125B model), chosen by the router: Strata feature (tech.hub77a.com),
 *     summary table row "핵심 기법" and section "2. 왜 대단한가" (1);
 *   - the compute path branches on the routing result: resident experts are
 *     used at once, the rest are first moved in from host memory: ibid. (2);
 *     Janas-LLM item (onedev.kr/items/2196): repeat experts stay cached;
 *   - a draft-and-verify step checks 1 + d guessed tokens in one pass, and the
 *     prompt path reads up to 8,192 tokens per chunk: Strata feature (3);
 *   - 2-bit class weights (Q2_0) are the fast size: Strata feature, section
 *     "3. 바로 써먹기", speed table.
 *
 * Weight format (b = 2, 3 or 4).  A matrix [R x K] (K % 32 == 0) is split
 * into blocks of 32 weights along K.  Each block carries an IEEE binary16
 * scale s and min m; weight = s * q + m for the block's b-bit unsigned codes q.
 *   code plane: row r is K*b/32 little-endian uint32 words.  b = 2, 4: word w
 *     holds columns w*(32/b) ... (w+1)*(32/b) - 1; column c of a word sits at
 *     bit 16*(c % 2) + b*(c / 2), so even columns fill the low halfword and
 *     odd columns the high halfword.  b = 3: three words per block; words 0
 *     and 1 hold the low two bits of the block's codes exactly as the b = 2
 *     layout holds codes, word 2 holds the high bit of block column j at bit
 *     16*(j % 2) + j / 2 (q = low + 4 * high);
 *   s/m plane: row r is K/32 uint32 words, scale in bits 0-15, min in 16-31;
 *   expert blob: Wg codes, Wg s/m, Wu codes, Wu s/m, Wd codes, Wd s/m, each
 *     plane starting on a 256-byte boundary; Wg and Wu are [I x H], Wd is
 *     [H x I]; the blob is moe_expert_bytes(H, I, b) bytes.
 *
 * Conventions for every call:
 *   - Pointers are device memory owned by the caller unless marked "host".
 *     The library never allocates device memory; scratch space is passed in
 *     and sized by the *_workspace_bytes queries.
 *   - Work is enqueued on the given stream and runs asynchronously; inputs
 *     must stay valid until the stream reaches it.  Nothing blocks the host
 *     except moe_slot_table_resolve/preload, which say so.
 *   - Arguments are checked on the host before anything is enqueued; a call
 *     that returns an error has enqueued nothing.  moe_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *   - A HIP runtime or launch failure is reported as MOE_EHIP.
 *   - Limits: 1 <= E <= 1024, 1 <= k <= min(16, E), H % 32 == 0 and
 *     I % 32 == 0 with 32 <= H <= 16384 and 32 <= I <= 8192, b in {2, 3, 4},
 *     T >= 0 (T == 0 enqueues nothing and returns MOE_OK).
 *   - Device buffers that the kernels read with 128-bit loads (expert blobs,
 *     activations) must be 16-byte aligned; the expert stride must be a
 *     multiple of 256.
 *   - Logits must be finite; NaN or infinite logits give unspecified (but
 *     memory-safe) routing.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* a null pointer, a negative size, inconsistent sizes */
  MOE_EUNSUPPORTED = 2, /* sizes outside the limits above */
  MOE_EWORKSPACE = 3,   /* the workspace is smaller than the query returned */
  MOE_EHIP = 4,         /* a HIP runtime or kernel launch error */
  MOE_ENOTPINNED = 5,   /* a host buffer that must be page-locked is not */
  MOE_ECAPACITY = 6     /* the slot table cannot hold the active set */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Which expert-FFN kernels to run.  AUTO picks GEMV for T * k <= 128 routed rows
 * and MFMA above (the measured crossover on the 512-expert, top-10 decode layer);
 * the arithmetic, and with it the tolerance a caller can expect (about 1e-5
 * against 5e-3 of a row's largest output), changes with the path. */
typedef enum moe_ffn_path {
  MOE_PATH_AUTO = 0,
  MOE_PATH_GEMV = 1, /* fused dequant-GEMV, fp32 throughout: decode and verify steps */
  MOE_PATH_MFMA = 2  /* weights decoded to fp16 in LDS, fp16 MFMA, fp32 accumulate: prefill */
} moe_ffn_path;

/* One layer's experts.  Expert e's blob is at base + idx(e) * stride where
 * idx(e) = slot_map[e] when slot_map is not NULL, else e.  slot_map (device,
 * [E]) is what a slot table maintains for one layer; an entry below zero
 * means "not resident" and makes that expert's output rows NaN. */
typedef struct moe_qlayer {
  int E, H, I, bits;
  const void* base;         /* device, 256-byte aligned */
  int64_t stride;           /* bytes, >= moe_expert_bytes(H, I, bits), multiple of 256 */
  const int32_t* slot_map;  /* device, NULL or [E] */
} moe_qlayer;

int moe_abi_version(void);
const char* moe_last_error(void);
const char* moe_status_string(moe_status st);

/* Bytes of one expert blob: 3*H*I*(b/8 + 4/32) plus plane padding to 256 B. */
size_t moe_expert_bytes(int H, int I, int bits);

/*
 * moe_route_topk -- top-k expert selection and gate weights.
 * Passage: Strata feature, summary row "핵심 기법" and section "2. 왜 대단한가"
 * (1)-(2) (the router picks a few experts per token and only those run).
 *   logits  [T x E] fp32, row-major.
 *   ids     [T x k] int32 out: the k largest logits of each row in descending
 *           order; equal logits rank the lower expert id first; -0.0 equals +0.0.
 *   w       [T x k] fp32 out: w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *           over the k selected logits (sums to 1 up to rounding).
 * Errors: MOE_EINVAL (null pointers with T > 0), MOE_EUNSUPPORTED (E, k out of range).
 */
moe_status moe_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t stream);

/*
 * moe_router_logits -- the router projection that produces the logits.
 * Passage: Strata feature, section "2. 왜 대단한가" (2) (the router's choice
 * decides which experts run).  The pages give no formula; the projection is a
 * bias-free linear map: logits[t][e] = sum_c x[t][c] * w_r[e][c].
 *   x       [T x H] device, fp32 or bf16 (x_t), row-major, 16-byte aligned.
 *   w_r     [E x H] device, bf16 bits (uint16), row-major, 16-byte aligned.
 *   logits  [T x E] fp32 out, row-major.
 * Products and sums in fp32 (a bf16 product is exact in fp32).  bf16 x with
 * T >= 64 runs a bf16 MFMA GEMM; otherwise one wave per expert row (a GEMV
 * over up to 16 tokens per pass).  No workspace.
 * Errors: MOE_EINVAL (null pointers with T > 0, T < 0, bad dtype),
 * MOE_EUNSUPPORTED (E, H out of the library limits).
 */
moe_status moe_router_logits(const void* x, moe_dtype x_t, const void* w_r, int T, int H, int E, float* logits,
                             hipStream_t stream);

/*
 * moe_router_topk -- moe_router_logits, then moe_route_topk on its logits.
 * logits is a caller buffer [T x E] fp32 that receives the logits; ids and w
 * as for moe_route_topk.  Two launches on `stream`.
 */
moe_status moe_router_topk(const void* x, moe_dtype x_t, const void* w_r, int T, int H, int E, int k, float* logits,
                           int32_t* ids, float* w, hipStream_t stream);

/*
 * moe_dispatch -- group the n = T*k assignments a = t*k + j by expert.
 * Passage: the tokens routed to one expert are computed together (Strata
 * feature, section "2. 왜 대단한가" (2): the compute path follows the routing).
 * The order is unique: ascending expert, and ascending a inside an expert.
 *   ids           [T x k] int32 in; ids outside [0, E) are dropped (not
 *                 counted, their assign_pos entry is -1).
 *   offsets       [E + 1] out: offsets[e] = number of kept assignments with expert < e.
 *   sorted_assign [n] out: the assignment at each sorted position (entries past
 *                 offsets[E] are left unchanged).
 *   assign_pos    [n] out: inverse of sorted_assign (-1 for dropped ones).
 *   active        [min(E, n)] out: experts with at least one assignment, ascending.
 *   n_active      [1] out: how many entries of active are set.
 *   ws            device scratch of at least moe_dispatch_workspace_bytes(T, k, E) bytes.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE.
 */
size_t moe_dispatch_workspace_bytes(int T, int k, int E);
moe_status moe_dispatch(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* active, int32_t* n_active, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * moe_expert_ffn_q -- SwiGLU FFN of every routed (token, expert) pair.
 * Passage: only the selected experts' weights are read (Strata feature,
 * section "2. 왜 대단한가" (1)); 2-bit class weights (speed table, section
 * "3. 바로 써먹기"); verify steps of 1 + d tokens and 8,192-token prompt
 * chunks (section "2. 왜 대단한가" (3)).
 * For each sorted position p in [offsets[e], offsets[e+1]) of each active
 * expert e, with a = sorted_assign[p] and t = a / k:
 *   g = Wg x[t], u = Wu x[t], h = silu(g) * u, y[a] = Wd h.
 *   x        [T x H], dtype x_t (MOE_F32 or MOE_BF16), 16-byte aligned.
 *   y        [T x k x H] out, dtype y_t; rows of dropped assignments are untouched.
 *   path     MOE_PATH_GEMV keeps g, u, h and the sums in fp32 (the bf16 dot
 *            instructions see x exactly, and fp32 values as a sum of two bf16
 *            parts); MOE_PATH_MFMA rounds the decoded weights, x and h to fp16
 *            and accumulates in fp32.  It first scales each token row of x by
 *            a power of two so that its largest magnitude lies in [1, 2), keeps
 *            h scaled by the square of its token's factor and undoes both after
 *            accumulation, so the fp16 range does not limit x or h; an h value
 *            still beyond +-65504 after that scaling saturates and is counted:
 *            once the call has completed, the first 4 bytes of ws hold that
 *            count as a uint32 (0 when nothing saturated).
 *   ws       device scratch of at least moe_expert_ffn_workspace_bytes(...) bytes.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE.
 */
size_t moe_expert_ffn_workspace_bytes(const moe_qlayer* q, int T, int k, moe_ffn_path path);
moe_status moe_expert_ffn_q(const moe_qlayer* q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                            const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                            moe_dtype y_t, moe_ffn_path path, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_combine -- weighted sum of the k expert rows of each token.
 * out[t][c] = residual[t][c] + sum_{j=0}^{k-1} w[t][j] * y[t][j][c], j ascending, fp32.
 *   y         [T x k x H], dtype y_t.
 *   w         [T x k] fp32 gate weights.
 *   residual  NULL or [T x H], dtype r_t.
 *   out       [T x H] fp32 out.
 *   out_bf16  NULL or [T x H] out: bf16 (round to nearest even) of out, as raw bits.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED.
 */
moe_status moe_combine(const void* y, moe_dtype y_t, const float* w, int T, int k, int H, const void* residual,
                       moe_dtype r_t, float* out, uint16_t* out_bf16, hipStream_t stream);

/*
 * moe_layer_decode -- the whole layer for decode and verify steps (T <= 12).
 * Passage: as for the four calls above (Strata feature, summary row "핵심 기법"
 * and section "2. 왜 대단한가" (1)-(3)).  Every output (ids, w, the dispatch
 * arrays, y, out, out_bf16) is bit-identical to moe_route_topk + moe_dispatch +
 * moe_expert_ffn_q(MOE_PATH_GEMV) + moe_combine on the same inputs.
 * Launches: when H is a multiple of 2048 and I of 512, two: the gate/up +
 * SwiGLU kernel, each of whose workgroups routes the T tokens itself (one of
 * them also writes ids, w and the dispatch arrays), then the down kernel with
 * the combine folded in.  Other shapes take four: routing, grouping and the
 * per-expert descriptors in one workgroup; gate/up + SwiGLU; down; combine.
 *   logits [T x E] fp32; x [T x H] (MOE_F32 or MOE_BF16); residual NULL or [T x H].
 *   Outputs as in the four calls; ws of moe_layer_decode_workspace_bytes bytes.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED (T > 12 or the limits above), MOE_EWORKSPACE.
 */
size_t moe_layer_decode_workspace_bytes(const moe_qlayer* q, int T, int k);
moe_status moe_layer_decode(const moe_qlayer* q, const float* logits, const void* x, moe_dtype x_t, int T, int k,
                            const void* residual, moe_dtype r_t, int32_t* ids, float* w, int32_t* offsets,
                            int32_t* sorted_assign, int32_t* assign_pos, int32_t* active, int32_t* n_active, void* y,
                            moe_dtype y_t, float* out, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * moe_layer_decode_noalloc -- moe_layer_decode without a caller workspace, for
 * callers that cannot allocate device memory or pass one in (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation).  The workspace is a fixed array of
 * moe_layer_decode_noalloc_max_bytes() bytes (1 MiB) in this library's device
 * code, one per GPU, held until the process ends; the call allocates nothing.
 * Steps whose moe_layer_decode_workspace_bytes exceeds it return
 * MOE_EUNSUPPORTED (the 512-expert, top-10, 2048 x 512 layer needs about
 * 0.2 MB at T = 3 and 0.8 MB at T = 12).  Arguments, outputs and errors are
 * those of moe_layer_decode, whose kernels it runs, and every output is
 * bit-identical to it.  All calls on one GPU share that GPU's array: calls
 * that can overlap on one GPU (several streams, several host threads) race and
 * must be ordered by the caller.  The first call on a device looks the array
 * up with that device current.
 */
size_t moe_layer_decode_noalloc_max_bytes(void);
moe_status moe_layer_decode_noalloc(const moe_qlayer* q, const float* logits, const void* x, moe_dtype x_t, int T,
                                    int k, const void* residual, moe_dtype r_t, int32_t* ids, float* w,
                                    int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* active,
                                    int32_t* n_active, void* y, moe_dtype y_t, float* out, uint16_t* out_bf16,
                                    hipStream_t stream);

/*
 * Resident-expert slot table.
 * Passage: the most-called experts stay resident in GPU memory while all of
 * them sit in host RAM; a routed expert that is resident is used at once and
 * any other is first moved in (Strata feature, section "2. 왜 대단한가" (2));
 * repeat experts are kept cached (Janas-LLM item); part of host memory is
 * locked for the graphics card (Strata feature, section "3. 바로 써먹기").
 *
 * The table manages n_slots device slots of expert_bytes each for the L*E
 * (layer, expert) blobs whose master copies sit in page-locked host memory:
 * blob (l, e) at host_experts + (l*E + e) * expert_bytes.  slot_map[l*E + e]
 * (device) holds the slot of (l, e) or -1.  Pass slots as moe_qlayer.base,
 * expert_bytes as .stride and slot_map + l*E as .slot_map.
 * Policy: least recently used over (layer, expert); misses of one resolve
 * are served in ascending expert order; a slot used by the same resolve is
 * never a victim.  The policy changes only timing, never results.
 * Copies and map updates are enqueued on the given stream, so kernels that
 * follow on that stream see them.  A table serves one stream and one host
 * thread at a time.
 */
typedef struct moe_slot_table moe_slot_table;

typedef struct moe_slot_stats {
  uint64_t hits, misses, bytes_h2d, resolves, evictions;
} moe_slot_stats;

/* MOE_ENOTPINNED when host_experts is not page-locked host memory;
 * expert_bytes must be a multiple of 256; slots and slot_map are device memory
 * of n_slots * expert_bytes bytes and L*E int32.  The map is set to -1 on
 * `stream` (enqueued; ordered before later work on it). */
moe_status moe_slot_table_create(int L, int E, int n_slots, size_t expert_bytes, const void* host_experts, void* slots,
                                 int32_t* slot_map, hipStream_t stream, moe_slot_table** out);

/* Make the given (layer, expert) pairs resident (host array of 2*n int32:
 * layer, expert, ...), in order, evicting least recently used slots.  Waits
 * for earlier work on stream (the slots and the map may still be in use),
 * then enqueues the copies and the map update on stream. */
moe_status moe_slot_table_preload(moe_slot_table* t, const int32_t* layer_expert, int n, hipStream_t stream);

/* Make every expert in active[0 .. *n_active) of `layer` resident.  active and
 * n_active are device arrays written earlier on `stream` (moe_dispatch); this
 * call copies them to the host and waits for them (it blocks the host until
 * the stream has reached this point), then enqueues the miss copies and the
 * map update on stream.  MOE_ECAPACITY if n_active > n_slots. */
moe_status moe_slot_table_resolve(moe_slot_table* t, int layer, const int32_t* active, const int32_t* n_active,
                                  hipStream_t stream);

moe_status moe_slot_table_stats(const moe_slot_table* t, moe_slot_stats* out);

/* Host view of the map: out (host, [L*E]) = slot of each (layer, expert) or -1.
 * In device mode the map is copied from the device with a blocking copy: call
 * it after the table's stream has finished (likewise moe_slot_table_stats). */
moe_status moe_slot_table_map_host(const moe_slot_table* t, int32_t* out);

/*
 * Device mode: the same policy run on the GPU, so that a resolve needs no host
 * round trip and can be captured in a graph (passage as above: the compute path
 * branches on the routing result and moves only the missing experts in).
 * moe_slot_table_enable_device moves the table's current state (after any
 * preload) into `state`, device memory of moe_slot_table_device_bytes bytes,
 * 256-byte aligned, owned by the caller and kept alive with the table; it
 * waits for `stream` and uploads with blocking copies.  From then on only
 * moe_slot_table_resolve_device may change the table (resolve and preload
 * return MOE_EINVAL).  host_experts must have a device mapping (page-locked
 * memory from hipHostMalloc has one).
 * moe_slot_table_resolve_device enqueues, on `stream`, one kernel that applies
 * the policy to active[0 .. *n_active) (device arrays, e.g. from moe_dispatch)
 * and one that copies the missed blobs from host_experts into their slots, so
 * kernels that follow on `stream` see the updated slots and map.  max_active
 * bounds *n_active (e.g. min(E, T*k)); MOE_ECAPACITY if max_active > n_slots.
 * Maps, copies and counters equal those of moe_slot_table_resolve on the same
 * sequence of active sets.
 */
size_t moe_slot_table_device_bytes(int L, int E, int n_slots);
/*
 * moe_layer_decode_slots -- moe_layer_decode through a slot table in device
 * mode: the routing workgroup also resolves the routed experts of `layer`
 * (moe_slot_table_resolve_device's policy), then the gate/up and down kernels
 * run on the slots.  Strata feature (tech.hub77a.com), section
 * "2. 왜 대단한가" (2): resident experts are used at once while the missing
 * ones move in from host RAM.  When H % 2048 == 0 and I % 512 == 0 the step
 * is two launches: in the gate/up launch one workgroup
 * routes and resolves and publishes the outcome through the table's device
 * state, the workgroups of resident experts run at once, and those of missed
 * experts wait for it, then read their gate/up rows from the master copy and
 * write them into the new slot as they are used, while other workgroups of
 * the grid copy the rest of each missed blob; the down launch (combine
 * folded) also writes the table's map, miss list and counters.  Other shapes
 * route and resolve in a launch of their own, then copy the misses in a
 * launch of their own or inside gate/up (four launches, or five when the
 * combine cannot be folded).  Two calls on one table must not overlap (one
 * stream).  q must be the table's view of `layer`:
 * base = slots, stride = expert_bytes, slot_map = map + layer * E.  Outputs
 * and workspace as moe_layer_decode (moe_layer_decode_workspace_bytes); every
 * output is bit-identical to moe_layer_decode on resident weights.
 * Errors: as moe_layer_decode; MOE_EINVAL if the table is not in device mode
 * or q is not its view of `layer`; MOE_ECAPACITY if min(E, T*k) > n_slots.
 */
moe_status moe_layer_decode_slots(const moe_qlayer* q, moe_slot_table* t, int layer, const float* logits,
                                  const void* x, moe_dtype x_t, int T, int k, const void* residual, moe_dtype r_t,
                                  int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* assign_pos, int32_t* active, int32_t* n_active, void* y, moe_dtype y_t,
                                  float* out, uint16_t* out_bf16, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_slot_table_enable_device(moe_slot_table* t, void* state, size_t state_bytes, hipStream_t stream);
moe_status moe_slot_table_resolve_device(moe_slot_table* t, int layer, const int32_t* active,
                                         const int32_t* n_active, int max_active, hipStream_t stream);

void moe_slot_table_destroy(moe_slot_table* t);

/*
 * Kernel timing hook (for measurement tools; not part of the layer).  The
 * next launch of `kernel` issued by this host thread is made with
 * hipExtLaunchKernel so that `start` and `stop` (created by the caller with
 * hipEventCreate) record the start and end of that kernel's execution on its
 * stream.  One request is pending at a time; a new call replaces it.
 */
typedef enum moe_kernel {
  MOE_KERNEL_ROUTE = 0,
  MOE_KERNEL_DISPATCH = 1,
  MOE_KERNEL_GEMV_GATEUP = 2, /* decode gate/up + SwiGLU */
  MOE_KERNEL_GEMV_DOWN = 3,   /* decode down GEMV */
  MOE_KERNEL_DECODE_PREP = 7, /* descriptor preparation of the stand-alone GEMV path */
  MOE_KERNEL_MFMA_GATEUP = 4,
  MOE_KERNEL_MFMA_DOWN = 5,
  MOE_KERNEL_COMBINE = 6,
  MOE_KERNEL_ROUTER = 8 /* router projection (GEMV or MFMA) */
} moe_kernel;
moe_status moe_profile_next_launch(moe_kernel kernel, hipEvent_t start, hipEvent_t stop);

/*
 * Host-only slot table for exercising the policy without a GPU.  Every copy
 * the real table would enqueue is reported to copy_fn(user, slot, layer,
 * expert) instead; resolve takes a host array of active experts.
 */
typedef void (*moe_copy_fn)(void* user, int slot, int layer, int expert);
moe_status moe_slot_table_create_host(int L, int E, int n_slots, moe_copy_fn copy_fn, void* user,
                                      moe_slot_table** out);
moe_status moe_slot_table_resolve_host(moe_slot_table* t, int layer, const int32_t* active, int n_active);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
