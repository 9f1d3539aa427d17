/*
 * caat_pcr.h -- C ABI of the MI355X (gfx950) partial channel-reduce library.
 *
 * Method: "Tensor-Parallelism with Partially Synchronized Activations"
 * (CAAT-Net; Lamprecht, Karnieli, Hanani, Giladi, Soudry, NeurIPS 2025,
 * arXiv 2506.19645), Introduction.  In tensor parallelism each of T ranks
 * computes a partial activation with its row-parallel linear layer
 * (attention out-projection, MLP down-projection); the usual all-reduce sums
 * those partials.  The partial channel-reduce sums only the hidden channels
 * of a sync set S and leaves every other channel with the rank's own value,
 * so ranks hold different activations afterwards.  No channel synced is an
 * ensemble of independent ranks; all channels synced is the ordinary layer.
 *
 * The T ranks are T shards resident in one GPU's memory:
 *   X   [T, M, Kr]  bf16   rank t's input slice (Kr = K / T features)
 *   W   [T, Kr, H]  bf16   rank t's weight slice
 *   mask[H]         uint8  nonzero = channel c is in S (the mask is S; the
 *                          fraction p of the paper is |S| / H)
 *   out [T, M, H]   bf16   rank t's activation after the partial reduce
 * All arrays are dense row-major (last index contiguous).  bf16 values are
 * passed as their raw 16-bit patterns.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller; the library keeps no
 *     reference after the call returns and allocates nothing.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream) and runs asynchronously; nothing synchronises or prints.
 *   - Arguments are validated on the host before any GPU work is enqueued; on
 *     an error nothing is enqueued and the status code says why.
 *   - Sizes: 1 <= T <= 64; M >= 0 (M == 0 enqueues nothing, and tensors
 *     with no elements may then be NULL); Kr and H are positive multiples of
 *     8; one rank's slices (M*Kr, Kr*H, M*H elements) stay below 2^30.
 *     Tensor pointers must be 16-byte aligned, the mask 8-byte aligned.
 *   - Sums of synced channels are taken in fp32, in ascending rank order,
 *     once per element, and the one result is written to every rank, so the
 *     synced channels are bit-identical across ranks and run to run.
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef CAAT_PCR_H
#define CAAT_PCR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CAAT_OK = 0,
  CAAT_ERR_NULL = 1,      /* a required pointer is NULL */
  CAAT_ERR_DIM = 2,       /* a size is out of range or not a multiple of 8 */
  CAAT_ERR_ALIGN = 3,     /* a pointer is misaligned */
  CAAT_ERR_ALIAS = 4,     /* an output overlaps an input (or another output) */
  CAAT_ERR_DTYPE = 5,     /* unknown dtype code */
  CAAT_ERR_WORKSPACE = 6, /* workspace missing or smaller than required */
  CAAT_ERR_LAUNCH = 7     /* the HIP runtime rejected a kernel launch */
} caat_status;

typedef enum { CAAT_F32 = 0, CAAT_BF16 = 1 } caat_dtype;

/* Version of this ABI (incremented on incompatible change). */
int caat_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* caat_status_string(int status);

/*
 * Forward: row-parallel linear layer followed by the partial channel-reduce
 * (Introduction of the paper):
 *   Y_t = X_t W_t                      (bf16 products, fp32 accumulation)
 *   out[t][:, c] = sum_u Y_u[:, c]     for c in S   (same value on every rank)
 *   out[t][:, c] = Y_t[:, c]           for c not in S
 * rounded once to bf16 (nearest even).  `out` must not overlap X, W or mask.
 * Three kernels serve it, by shape:
 *   - few tokens (H <= 65536; M <= 32 with T <= 8, M < 24 with more ranks;
 *     with T = 1, M <= 192, 32 tokens at a time): a weight-streaming kernel
 *     whose workgroups exchange fp32 partials of the synced channels through
 *     the workspace.  With few ranks or channels each rank's contraction is
 *     cut into ks slices of whole 32-row stages (ks doubled while
 *     T * ks <= 8, T * ceil(H/128) * ks <= 256 and ceil(Kr/32) >= 16 * ks),
 *     every slice's fp32 partials go through the workspace, and each rank's
 *     value is its slices' sum in slice order;
 *   - from there on, T >= 2, while the fused kernel below would have few tiles for
 *     its walk over the ranks (ceil(H/128) * ceil(M/64) at most
 *     3 * T * ceil(Kr/64) + 128 with T <= 8, 2 * T * ceil(Kr/64) + 64 with
 *     more, 128 when Kr <= 128): one workgroup per (rank, tile of 128
 *     channels x 64 or 128 tokens, or 256 x 256 when those fill whole rounds
 *     of the 256 CUs and their token blocks at least 3/4) writes fp32
 *     products Y[T,M,H] into the workspace, and a
 *     streaming pass reduces them into out (the synced sum is the
 *     ascending-rank fp32 sum of the per-rank products; with whole
 *     contractions and H a multiple of 64, 64-channel groups with no synced
 *     channel go straight to out and skip the pass).  With at most 256
 *     tiles of 128 x 64 and at least 16 chunks of 64 in each rank's
 *     contraction, that contraction is cut in two slices whose fp32 products
 *     (twice the workspace) are added first;
 *   - otherwise the fused tile kernel (each tile walks all T ranks), which
 *     needs no workspace.  With 2 <= T <= 8 and short contractions (at most
 *     six chunks of 64 per rank, twelve with the smallest tiles) it runs in
 *     two launches: 256-channel groups of the mask whose 8-channel chunks
 *     mix synced and local channels go to a variant that holds the earlier
 *     ranks' tiles in registers and writes each output line once.
 * caat_rowpar_pcr_fwd_workspace_bytes() gives the bytes a call needs (0:
 * pass NULL, 0).  The workspace starts with a 2 KiB region of 32-bit arrival
 * counters (the same size and place for every shape) that must be zero when
 * a call starts; every call leaves them zero again, so zero a new workspace
 * once before its first use and it stays valid for calls of any later
 * shape.  The rest (from byte 2048 on) may hold anything.  Every path gives
 * the same value up to fp32 summation order; for a given shape and workspace
 * the bits are fixed.
 */
int caat_rowpar_pcr_fwd(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out,
                        int T, int M, int Kr, int H,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t caat_rowpar_pcr_fwd_workspace_bytes(int T, int M, int Kr, int H);

/*
 * caat_rowpar_pcr_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with no workspace argument.
 * Calls that need a workspace use a scratch area owned by the library
 * instead, a static device array of CAAT_NOALLOC_SCRATCH_BYTES (16 MiB) on
 * each GPU, held until the process ends.  A split-path call whose fp32
 * products would exceed it cuts the contraction into fewer slices, or, if
 * even whole contractions do not fit, runs the path the shape would take
 * without the split (chunked decode or fused tiles); either gives the same
 * value up to fp32 summation order.  A decode call whose partials exceed it
 * (e.g. T*H > 131056 channels over all ranks at M = 32, whole contractions;
 * calls in contraction slices need at most 4 MiB and always fit) returns
 * CAAT_ERR_WORKSPACE before anything is enqueued.  The scratch of the device
 * current at the call is used (`stream` must belong to it); its arrival
 * counters are cleared by the call itself (a small fill kernel, no memset).
 * Every call on one GPU shares that GPU's scratch, so calls that may overlap
 * on one GPU (different streams, different threads) race and must be
 * serialised by the caller.  Calls that need no workspace behave exactly like
 * caat_rowpar_pcr_fwd, and so do the others whose workspace fits the
 * scratch.  Neither call allocates; this one calls no hipMalloc, hipFree or
 * allocating library routine at all.  CAAT_ERR_LAUNCH also covers a failed
 * lookup of the scratch's device address.
 */
#define CAAT_NOALLOC_SCRATCH_BYTES (16u << 20)
int caat_rowpar_pcr_fwd_noalloc(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out,
                                int T, int M, int Kr, int H, void* stream);

/*
 * Backward of caat_rowpar_pcr_fwd for per-rank incoming gradients dZ[T,M,H]
 * (bf16).  The partial channel-reduce is linear and self-adjoint, which is
 * the forward/backward agreement the paper's Introduction requires:
 *   G_t[:, c] = sum_u dZ_u[:, c]  for c in S,   dZ_t[:, c]  for c not in S
 *   dX[t] = G_t W_t^T   [M, Kr] bf16      dW[t] = X_t^T G_t   [Kr, H] bf16
 * G's synced channels are rounded to bf16 once (they feed bf16 MFMA); both
 * products accumulate in fp32.  dX or dW may be NULL to skip that product.
 * Needs caat_pcr_bwd_workspace_bytes() bytes of workspace, any contents on
 * entry and unspecified contents on return: T*M*H*2 (rounded up to 256) for
 * G[T,M,H] (bf16), then 256 bytes, plus, when dW's tiles cannot fill the
 * chip's 256 CUs and M spans at least 16 chunks of 64 tokens, s*T*Kr*H*4
 * bytes after those for dW's fp32 sums over s pieces of the token range
 * (added in piece order, so the result does not depend on scheduling).
 * With H <= 16384, G is only written where it differs from dZ per rank:
 * 256-channel tiles with no synced channel are read from dZ directly, and
 * tiles whose channels are all synced hold the one sum once (a contiguous S
 * then forms a fraction p of G instead of all of it); the results are the
 * same.
 * Outputs must not overlap the inputs, the workspace or each other.
 */
int caat_pcr_bwd(const uint16_t* dZ, const uint16_t* X, const uint16_t* W, const uint8_t* mask,
                 uint16_t* dX, uint16_t* dW, int T, int M, int Kr, int H,
                 void* workspace, size_t workspace_bytes, void* stream);
size_t caat_pcr_bwd_workspace_bytes(int T, int M, int Kr, int H);

/*
 * Column-parallel linear layer with per-rank inputs: the layer that consumes
 * the partial channel-reduce's output.  After the partial reduce the ranks'
 * activations differ (paper, Introduction), so rank t multiplies its own
 * activation A_t by its own column slice W_t of the next layer's weight:
 *   A [T, M, K] bf16   rank t's activation (K = the hidden size)
 *   W [T, K, N] bf16   rank t's column slice (N output columns per rank)
 *   U [T, M, N] bf16   U[t] = A_t W_t   (fp32 accumulation, rounded once)
 * Sizes and alignment as above with (Kr, H) = (K, N).  No workspace; U must
 * not overlap A or W.
 */
int caat_colpar_fwd(const uint16_t* A, const uint16_t* W, uint16_t* U, int T, int M, int K, int N,
                    void* stream);

/*
 * Backward of caat_colpar_fwd for per-rank incoming gradients dU[T,M,N]:
 *   dA[t] = dU_t W_t^T   [M, K] bf16      dW[t] = A_t^T dU_t   [K, N] bf16
 * (fp32 accumulation).  Each rank's input gradient stays on its rank: an
 * ordinary tensor-parallel backward sums the column-parallel layer's input
 * gradient over the ranks because that input is replicated, but here the
 * inputs differ and the only cross-rank sum is the partial channel-reduce's
 * own backward (caat_pcr_bwd with dZ = dA), over exactly the synced
 * channels -- the forward/backward agreement the Introduction requires.
 * dA or dW may be NULL to skip that product.  No workspace; outputs must not
 * overlap the inputs or each other.
 */
int caat_colpar_bwd(const uint16_t* dU, const uint16_t* A, const uint16_t* W, uint16_t* dA, uint16_t* dW,
                    int T, int M, int K, int N, void* stream);

/*
 * The step after the partial channel-reduce in the Llama-family blocks the
 * paper trains (reproducibility table: Llama2-7B, TinyLlama-1.1B): each rank
 * adds its own activation Z_t -- rank-specific after the partial reduce
 * (Introduction) -- to its own residual stream R_t and RMS-normalises the
 * result with the norm weight gamma (the same on every rank):
 *   Rout[t,m,:] = bf16(R[t,m,:] + Z[t,m,:])
 *   N[t,m,:]    = bf16(Rn * gamma / sqrt(mean_c Rn^2 + eps)),  Rn = the rounded Rout row
 * in fp32; the row's sum of squares is formed in a fixed order, so results
 * are bitwise reproducible.  Z, R, Rout, N [T,M,H] bf16; gamma [H] bf16;
 * 0 <= eps (finite).  H <= 8192.  Rout == R updates the residual stream in
 * place; otherwise Rout must not overlap Z, R or gamma.  N must not overlap
 * any other argument.  No workspace.
 */
int caat_residual_rmsnorm(const uint16_t* Z, const uint16_t* R, const uint16_t* gamma, uint16_t* Rout,
                          uint16_t* N, int T, int M, int H, float eps, void* stream);

/*
 * The partial channel-reduce with the step after it fused into its epilogue
 * (paper, Introduction: after the partial reduce each rank's activation is
 * its own and feeds its own residual stream; the Llama-family blocks of the
 * reproducibility table then RMS-normalise it).  For per-rank bf16 partial
 * activations Y[T,M,H] (the row-parallel products before the reduce):
 *   Z_t     = the partial channel-reduce of Y, as caat_partial_channel_reduce
 *             with CAAT_BF16 (synced channels: fp32 sum in ascending rank
 *             order, rounded once; local channels: Y_t)
 *   Rout[t] = bf16(R[t] + Z_t)
 *   N[t]    = bf16(Rout row * gamma / sqrt(mean(Rout row^2) + eps))
 * Z is never written: one pass reads Y and R and writes Rout and N, the same
 * bits as caat_partial_channel_reduce followed by caat_residual_rmsnorm.
 * Y, R, Rout, N [T,M,H] bf16; mask [H] uint8; gamma [H] bf16; 0 <= eps
 * (finite); H <= 8192; one rank's slice M*H below 2^30 elements.
 * Rout == R updates the residual stream in place; otherwise Rout must not
 * overlap R.  Neither output may overlap Y, mask or gamma, and N may not
 * overlap R or Rout.  No workspace.
 */
int caat_partial_channel_reduce_residual_rmsnorm(const uint16_t* Y, const uint8_t* mask, const uint16_t* R,
                                                 const uint16_t* gamma, uint16_t* Rout, uint16_t* N,
                                                 int T, int M, int H, float eps, void* stream);

/*
 * The partial channel-reduce alone, on given per-rank activations Y[T,M,H]
 * of `dtype` (CAAT_F32 or CAAT_BF16):
 *   out[t][:, c] = Y[0][:, c] + Y[1][:, c] + ... + Y[T-1][:, c]   for c in S
 *   out[t][:, c] = Y[t][:, c]                                      for c not in S
 * (fp32 sum in that order; bf16 rounds the sum once).  out == Y runs in
 * place and never writes the local channels; otherwise out must not overlap Y.
 * As for every call, one rank's slice M*H must stay below 2^30 elements
 * (CAAT_ERR_DIM otherwise).
 */
int caat_partial_channel_reduce(const void* Y, const uint8_t* mask, void* out,
                                int T, int M, int H, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAAT_PCR_H */
