/*
 * trimul.h -- C ABI of the MI355X (gfx950) triangle multiplicative update.
 *
 * The operation is the one defined on the page "Triangle Multiplicative Update
 * (SM100 / SM103 / SM107)", section "Mathematics and numerics": for every pair
 * (i, j) of a batch entry, with pair mask m,
 *
 *   z_in = LayerNorm_{c_z}(x; norm_in_weight, norm_in_bias, eps)
 *   a    = sigmoid(z_in g_in[:c]^T + g_in_b[:c]) * (z_in p_in[:c]^T + p_in_b[:c]) * m
 *   b    = sigmoid(z_in g_in[c:]^T + g_in_b[c:]) * (z_in p_in[c:]^T + p_in_b[c:]) * m
 *   y    = sum_k a[i,k] * b[j,k]   (outgoing)   or   sum_k a[k,i] * b[k,j]   (incoming)
 *   u    = LayerNorm_c(y; norm_out_weight, norm_out_bias, eps)
 *   out  = sigmoid(z_in g_out^T + g_out_b) * (u p_out^T + p_out_b)
 *
 * forward only, bf16 storage with fp32 arithmetic, rounding once to bf16 at
 * z_in and u (the matrix-core operands), at a and b (after the mask multiply,
 * a zero mask gives +0.0), at y, and at out. The output is not masked; the
 * residual add is the caller's.
 *
 * Every tensor is a bf16 DEVICE pointer, contiguous, row-major, 16-byte
 * aligned, on the current HIP device:
 *   x               [B, N, N, c_z]   pair representation
 *   mask            [B, N, N]        pair mask (NULL = every pair valid)
 *   norm_in_w/_b    [c_z]            LayerNorm_in affine (required)
 *   p_in_w, g_in_w  [2c, c_z]        rows [a; b] (required)
 *   p_in_b, g_in_b  [2c]             (optional, NULL = 0)
 *   norm_out_w/_b   [c]              LayerNorm_out affine (required)
 *   p_out_w         [c_z, c]         (required)
 *   g_out_w         [c_z, c_z]       (required)
 *   p_out_b, g_out_b [c_z]           (optional, NULL = 0)
 *   out             [B, N, N, c_z]   written, never read
 * (parameter conventions: same page, same section.)
 *
 * Ownership: the caller owns every buffer. The library allocates nothing on
 * the device and never synchronizes the stream; work is enqueued on `stream`
 * (a hipStream_t; NULL = the null stream). out and the workspace must not
 * overlap, as byte ranges, any tensor the kernels read or each other (the
 * output stage reads x while it writes out). All checks happen before any
 * launch; on error nothing is enqueued.
 *
 * Supported envelope (same page, section "Served today, and the typed
 * declines", re-targeted to gfx950): c_z == c in {128, 256}; any N >= 1 in
 * either direction; B >= 1; B*N*N*c_z and 2*c*B*N*n_pad below 2^31
 * (32-bit element offsets inside the kernels).
 */
#ifndef TRIMUL_H
#define TRIMUL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define TRIMUL_OK 0
#define TRIMUL_E_INVALID 1      /* bad argument: direction, NULL required weight, alignment,
                                   aliasing, workspace too small, c_z % 32 != 0, eps */
#define TRIMUL_E_UNSUPPORTED 2  /* outside the kernels' envelope: device is not gfx950,
                                   c_z != c or c not in {128, 256}, extent >= 2^31 */
#define TRIMUL_E_DEVICE 3       /* HIP runtime / launch failure */

/* Directions (same page, "Overview": the outgoing and incoming triangle
 * multiplications). */
#define TRIMUL_OUTGOING 0
#define TRIMUL_INCOMING 1

/* Library version string (static storage). */
const char* trimul_version(void);

/* Message of the last failing call on this thread (static, thread-local storage;
 * "" after a successful call). Names the rule and the operands involved. */
const char* trimul_last_error(void);

/* The padded inner length of the channel-major planes: N rounded up to a
 * multiple of 64 (same page, "Prepared class API", pads the inner axis to a
 * multiple of 8; a multiple of 64 here lets the contraction's k steps and the
 * 64-pair tiles of the other stages run without a tail). */
int trimul_n_pad(int N);

/* Workspace bytes for one call: three channel-major bf16 planes a, b and y,
 * each [c, B*N, n_pad] and each starting at a 256-byte aligned offset (same
 * page, "Overview" and "Prepared class API"). Layout, from the workspace base:
 *   a at 0, b at P, y at 2P, with P = round_up(c*B*N*n_pad*2, 256).
 * Plane element (ch, r, s) is at ch*B*N*n_pad + r*n_pad + s with r = b*N + i.
 *   outgoing: a(ch, b*N+i, k) = a[b,i,k,ch]    b(ch, b*N+j, k) = b[b,j,k,ch]
 *   incoming: a(ch, b*N+i, k) = a[b,k,i,ch]    b(ch, b*N+j, k) = b[b,k,j,ch]
 *   both:     y(ch, b*N+i, j) = y[b,i,j,ch]
 * Columns s in [N, n_pad) of a and b are written as +0.0; those of y hold
 * unspecified values. Returns 0 for arguments outside the envelope. */
size_t trimul_workspace_bytes(int B, int N, int c, int direction);

/* Typed support check with no launch (same page, "Served today, and the typed
 * declines"): widths, N, extent, direction, and -- when device >= 0 -- that
 * HIP device `device` is a gfx950. Returns a status code. */
int trimul_check_support(int B, int N, int c_z, int c, int direction, int device);

/* Every argument rule of trimul_forward, checked on the host only: no HIP call
 * is made, so pointer values are only compared (never dereferenced). Returns a
 * status code; the reason is in trimul_last_error(). */
int trimul_validate(const void* x, const void* mask,
                    const void* norm_in_w, const void* norm_in_b,
                    const void* p_in_w, const void* p_in_b,
                    const void* g_in_w, const void* g_in_b,
                    const void* norm_out_w, const void* norm_out_b,
                    const void* p_out_w, const void* p_out_b,
                    const void* g_out_w, const void* g_out_b,
                    int B, int N, int c_z, int c, int direction, float eps,
                    const void* out, const void* workspace, size_t workspace_bytes);

/* The forward pass (same page, "Overview": three launches on one stream).
 * Validates (as trimul_validate, plus the device check), then enqueues
 *   stage 1: LayerNorm_in + gated dual projection + mask -> planes a, b
 *   stage 2: per-channel contraction                      -> plane y
 *   stage 3: LayerNorm_out + LayerNorm_in recomputed + gated output projection -> out
 * on `stream`. Allocates nothing, does not synchronize. */
int trimul_forward(const void* x, const void* mask,
                   const void* norm_in_w, const void* norm_in_b,
                   const void* p_in_w, const void* p_in_b,
                   const void* g_in_w, const void* g_in_b,
                   const void* norm_out_w, const void* norm_out_b,
                   const void* p_out_w, const void* p_out_b,
                   const void* g_out_w, const void* g_out_b,
                   int B, int N, int c_z, int c, int direction, float eps,
                   void* out, void* workspace, size_t workspace_bytes, void* stream);

/* One stage of trimul_forward (stage = 1, 2 or 3), with the same arguments
 * and checks; calling stages 1, 2, 3 in order on one stream enqueues exactly
 * the work of trimul_forward. For per-stage timing and tests of the workspace
 * planes. */
int trimul_forward_stage(int stage,
                         const void* x, const void* mask,
                         const void* norm_in_w, const void* norm_in_b,
                         const void* p_in_w, const void* p_in_b,
                         const void* g_in_w, const void* g_in_b,
                         const void* norm_out_w, const void* norm_out_b,
                         const void* p_out_w, const void* p_out_b,
                         const void* g_out_w, const void* g_out_b,
                         int B, int N, int c_z, int c, int direction, float eps,
                         void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Allocation-free forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. ----
 *
 * The same computation, checks and kernels as trimul_forward, with the a, b
 * and y planes kept in a fixed device array inside the library instead of a
 * caller workspace: TRIMUL_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, reserved
 * when the library's device code is loaded on that GPU and held until the
 * process ends. The caller still passes every input and `out`. Calls whose
 * planes (trimul_workspace_bytes(B, N, c, direction)) exceed that size are
 * declined with TRIMUL_E_UNSUPPORTED before any launch (c = 128, B = 1 is
 * served up to N = 273; c = 256, B = 1 up to N = 192); use trimul_forward then.
 * No allocation and no synchronization happen on any call; the first call on
 * a device also reads the device's properties and looks up that device's copy
 * of the array (neither is a stream operation, but a capture that forbids
 * such calls would refuse them: make the first call on each device outside
 * any stream capture). The array keeps the last call's planes; no part of it needs to
 * start at zero. Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams or host threads without
 * ordering between them) race and give undefined results. */
#define TRIMUL_NOALLOC_SCRATCH_BYTES (64u << 20)

int trimul_forward_noalloc(const void* x, const void* mask,
                           const void* norm_in_w, const void* norm_in_b,
                           const void* p_in_w, const void* p_in_b,
                           const void* g_in_w, const void* g_in_b,
                           const void* norm_out_w, const void* norm_out_b,
                           const void* p_out_w, const void* p_out_b,
                           const void* g_out_w, const void* g_out_b,
                           int B, int N, int c_z, int c, int direction, float eps,
                           void* out, void* stream);

/* ---- Captured forward (same page, "Prepared class API": make_cuda_graph,
 * "one graph launch per call for these buffers"; the small-N calls are host
 * bound when launched eagerly). ----
 *
 * trimul_graph_create validates its arguments as trimul_forward does
 * (including the device check, on the current HIP device), then captures the
 * three stage launches for exactly these buffers into a HIP graph and
 * instantiates it. It allocates (a capture stream, the graph) and
 * synchronizes nothing on any caller stream; nothing runs until a launch. On
 * success *graph receives an opaque handle; on failure *graph is set to NULL.
 *
 * trimul_graph_launch enqueues one forward pass on `stream` (a stream of the
 * device the graph was created on; NULL = the null stream). The graph reads
 * the buffers' contents at launch time, so callers may rewrite x, the mask
 * and the parameters between launches; the buffers must stay allocated and
 * keep their sizes while the handle lives. Launches of one handle on
 * different streams must not overlap (they share the workspace).
 *
 * trimul_graph_destroy releases the handle (NULL is accepted). Work already
 * launched completes normally. */
typedef struct trimul_graph_s* trimul_graph_t;

int trimul_graph_create(const void* x, const void* mask,
                        const void* norm_in_w, const void* norm_in_b,
                        const void* p_in_w, const void* p_in_b,
                        const void* g_in_w, const void* g_in_b,
                        const void* norm_out_w, const void* norm_out_b,
                        const void* p_out_w, const void* p_out_b,
                        const void* g_out_w, const void* g_out_b,
                        int B, int N, int c_z, int c, int direction, float eps,
                        void* out, void* workspace, size_t workspace_bytes,
                        trimul_graph_t* graph);

int trimul_graph_launch(trimul_graph_t graph, void* stream);

int trimul_graph_destroy(trimul_graph_t graph);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_H */
