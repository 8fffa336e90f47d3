/*
 * q4.h -- C ABI of the GGUF Q4_0 hot-path library for AMD Instinct MI355X
 * (gfx950).
 *
 * What it computes.  The pages ("Implémentation en Rust du modèle Voxtral
 * Mini 4B Realtime de Mistral pour l'exécuter dans le navigateur", and its
 * es/id/hi copies) run the quantised speech model from a GGUF Q4_0 file:
 * section "Architecture" names the Q4_0 path and the encoder (width 1280) and
 * decoder (width 3072, GQA 32Q/8KV) whose projections it feeds; section
 * "Solutions techniques pour l'exécution dans le navigateur", item 3, keeps the
 * 131072-row token-embedding table as Q4 on the GPU with a row lookup.  Every
 * projection is y = deq(W) x, the LM head is its argmax, the embedding lookup
 * is a gather of decoded rows.
 *
 * Q4_0 layout (GGUF convention; the pages name the format but do not spell it
 * out).  A row of K weights (K a multiple of 32) is K/32 blocks of 18 bytes,
 * rows stored back to back (row stride 18*K/32 bytes).  Block: IEEE binary16
 * scale d, little-endian, in bytes 0-1; bytes 2..17 hold qs[0..15].  Weight j
 * of the block (j < 16) is the low nibble of qs[j], weight j+16 the high
 * nibble; its value is (q - 8) * d.  The byte array is used as stored, never
 * repacked.
 *
 * Conventions for every entry point below.
 *  - Pointers named w_q4, table_q4, x, r, y, out, ids, workspace are DEVICE
 *    pointers; the caller owns every buffer.  The library never allocates,
 *    frees or synchronises.
 *  - Outputs and workspaces overlap neither the inputs nor each other, except
 *    where an entry point allows it (q4_matmul_residual's r may be y;
 *    q4_decode_chain's x may lie inside an earlier step's y).
 *  - All device pointers must be 16-byte aligned (Q4_ERR_ALIGN otherwise).
 *  - Dense matrices are row-major and contiguous: x is [M, K] floats, y is
 *    [M, N] floats.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Each
 *    call only enqueues work on it and returns.
 *  - Arguments are validated before any HIP call; on a validation error
 *    nothing is enqueued.  A failed launch returns Q4_ERR_HIP and
 *    q4_last_hip_error() gives the hipError_t.  Values outside the documented
 *    ranges that live in device memory (token ids) cannot be checked on the
 *    host and are handled on the device as stated per call.
 *  - Calls are thread-safe; the only global state is a per-device cache of
 *    device properties.
 */
#ifndef Q4MI_Q4_H
#define Q4MI_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int q4_status;

enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,      /* a required pointer is NULL                        */
    Q4_ERR_SHAPE = 2,     /* M, N or K out of range, or K % 32 != 0            */
    Q4_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned           */
    Q4_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
    Q4_ERR_HIP = 5,       /* a HIP call failed; see q4_last_hip_error()        */
    Q4_ERR_FORMAT = 6,    /* a GGUF file is malformed or uses an unknown form  */
    Q4_ERR_IO = 7,        /* a file could not be opened or read                */
    Q4_ERR_NOT_FOUND = 8  /* no such tensor / metadata key / index             */
};

/* Version of this ABI (bumped on any incompatible change). */
int q4_abi_version(void);

/* Static text for a status code (never NULL). */
const char* q4_status_string(q4_status status);

/* hipError_t of the most recent Q4_ERR_HIP returned on the calling thread
 * (0 if none). */
int q4_last_hip_error(void);

/* Bytes of one Q4_0 row of K weights: 18*K/32.  Returns 0 if K is not a
 * positive multiple of 32. */
size_t q4_row_bytes(int64_t K);

/*
 * q4_matvec -- decode-step projection (the per-token decoder projections of
 * section "Architecture"): y[m, n] = sum_k deq(W)[n, k] * x[m, k].
 *   w_q4 : N rows of Q4_0, N*18*K/32 bytes.
 *   x    : [M, K] float32.    y : [M, N] float32 (written, not accumulated).
 *   1 <= M <= 8, N >= 1, K a positive multiple of 32, N*K < 2^40.
 * Float32 products of the exactly decoded, centred codes (q - 8) with x,
 * float32 accumulation, the block scale applied per block: the error stays
 * within 1e-4 * sum_k |w_k x_k| + 1e-6 for any finite x whose per-block sums
 * sum_j |q_j - 8| |x_j| stay below the float32 maximum (|x| < 1.3e36
 * always does; a zero weight, q = 8, adds exactly nothing whatever its x),
 * and results that fit in float32.  Tuned for M = 1.  With M >= 2 the rows of
 * x are taken in pairs: each pair's workgroups read and decode W once and
 * multiply it into both rows (K % 64 == 0, K <= 12288; otherwise each row
 * runs its own workgroups), so W is read ceil(M / 2) times (mostly from the
 * caches when W is small).  Results are deterministic (fixed reduction
 * order) and a row's result does not depend on the other rows of x: every
 * row has the bits it has in a call with that row alone.
 */
q4_status q4_matvec(const void* w_q4, const float* x, float* y,
                    int64_t M, int64_t N, int64_t K, void* stream);

/*
 * q4_matmul -- prefill / encoder projection (section "Architecture": encoder
 * width 1280, the 4x-downsample adapter, the decoder's 38/76-token prefix of
 * section "Correction du padding Q4"): Y = X * deq(W)^T.
 *   w_q4 : N rows of Q4_0.  x : [M, K] float32.  y : [M, N] float32.
 *   1 <= M <= 65535*128, 1 <= N < 2^31, K a positive multiple of 32 and at
 *   most 4194304.
 *   workspace, ws_bytes : optional device scratch (NULL allowed).  When the
 *             output tiles alone cannot fill the GPU, K is split over
 *             several workgroups whose float32 partial sums go to the
 *             workspace and are added in a fixed order by a second launch;
 *             q4_matmul_workspace_bytes(M, N, K) is the size that allows the
 *             planned split on the current device (0: no split planned).  A
 *             smaller workspace gives fewer splits (never an error).  Calls
 *             that share a workspace must be ordered.
 * M >= 5: activations are rounded to binary16 (round to nearest even) and
 * multiplied on the matrix cores with float32 accumulation, so |x| must stay
 * below 65504.  From 5 to 16 rows with K % 64 == 0 and K <= 6144 (a short
 * prefix, a few decode streams) the weights enter the matrix cores exactly
 * (q - 8, the block scale applied in float32), read once by a persistent
 * kernel with no K split; from 17 to 48 rows with K <= 3072 the same kernel
 * takes the decoded weights rounded to binary16.  Everywhere but on the
 * exact route the decoded weights are rounded to binary16, so every decoded
 * weight must stay below 65504: a block whose
 * scale exceeds 8188 in magnitude (largest |w| above 65504, which an encoder
 * only writes for weights that large) decodes to +-inf there.  M <= 4
 * (several decode streams) meets the q4_matvec bound, over q4_matvec's range
 * of x: either the rows of x go through the q4_matvec kernel (one row; two
 * rows unless K <= 3072 with 20 MiB of weights or more; K % 64 == 32; and,
 * for three or four rows with K > 6144, weights small enough that the rows'
 * repeated reads stay in the caches: (M - 1) * N * K * 18/32 bytes up to
 * 40 MiB, K <= 12288), or the weights are read once (by the persistent
 * stream16 kernel for three or four rows with K <= 6144 and for those two
 * rows, else by the small-M kernel) and enter the matrix cores
 * exactly (q - 8, block scale applied in float32) with x as two binary16
 * parts after a power-of-two scaling per 256-value chunk of a row;
 * a chunk whose nonzero magnitudes span more than 2^20 (or reach 2^124) is
 * summed in float32 instead, so no value of x loses its precision to the
 * scaling of a larger one.  Deterministic for
 * a given shape, device and ws_bytes; the split changes the order of the
 * float32 sums, so results for different workspace sizes may differ by
 * rounding.
 */
size_t q4_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);
q4_status q4_matmul(const void* w_q4, const float* x, float* y,
                    int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * q4_matmul_residual -- a projection with the residual add fused into its
 * epilogue (section "Architecture": in the encoder of width 1280 the
 * attention output and feed-forward down projections, 1280 outputs wide,
 * feed the residual stream): y = r + X * deq(W)^T.
 *   r : [M, N] float32 (device); either y itself (y += X deq(W)^T in
 *       place) or a buffer that does not overlap y.
 *   The other arguments are those of q4_matmul.
 * Bit for bit, y[m, n] = r[m, n] + p[m, n] rounded once in float32, where p
 * is what q4_matmul returns for the same arguments and workspace size.  The
 * add rides in a kernel of the product -- the wide kernel's stores (routes
 * "wide128" to "wide32" of q4_matmul_route, the encoder and adapter shapes)
 * or, with a K split, the fold -- and in a second launch after the finished
 * product on the other routes, where in place the product waits in the
 * workspace (M*N*4 bytes, else Q4_ERR_WORKSPACE).
 * q4_matmul_residual_workspace_bytes(M, N, K) covers every case on the
 * current device.
 */
size_t q4_matmul_residual_workspace_bytes(int64_t M, int64_t N, int64_t K);
q4_status q4_matmul_residual(const void* w_q4, const float* x, const float* r, float* y,
                             int64_t M, int64_t N, int64_t K,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * q4_embed_rows -- token-embedding lookup (section "Solutions techniques pour
 * l'exécution dans le navigateur", item 3): out[i, :] = deq(T[ids[i], :]).
 *   table_q4 : N rows of Q4_0 (N = vocabulary size, K = model width).
 *   ids      : M int32 token ids (device memory).
 *   out      : [M, K] float32; the decoded values are exact.
 *   M >= 1, N >= 1, K a positive multiple of 32.
 * An id outside [0, N) yields a row of zeros; the table is never read out of
 * bounds.
 */
q4_status q4_embed_rows(const void* table_q4, const int32_t* ids, float* out,
                        int64_t M, int64_t N, int64_t K, void* stream);

/*
 * q4_lmhead_argmax -- greedy next-token choice over the LM head (the same
 * 131072-row table read as a matrix): out_idx[m] = the lowest n attaining
 * max_n sum_k deq(T)[n, k] * x[m, k], out_val[m] that maximum (float32, same
 * arithmetic as q4_matvec).
 *   w_q4    : N rows of Q4_0.   x : [M, K] float32.
 *   out_idx : M int32 (device).  out_val : M float32 (device) or NULL.
 *   workspace, ws_bytes : device scratch of at least
 *             q4_lmhead_argmax_workspace_bytes(M, N, K) bytes (256 per row
 *             of x).  It must be zero before the first call; every call that
 *             completes leaves it zero again, so it can be reused without
 *             clearing.  Calls that share a workspace must be ordered (same
 *             stream or synchronised).
 * One launch: each workgroup folds its best (value, lowest index) into a
 * per-row key with a device-scope atomic max (order-independent, hence
 * deterministic); the last workgroup to finish writes the outputs and clears
 * the workspace.  On tables of 65536 rows or more with K <= 4096 the rows of
 * x are taken in pairs (the table is read once per pair); a row's index and
 * value are those of a call with that row alone.
 *   1 <= M <= 64, 1 <= N < 2^31, K a positive multiple of 32.
 * Logits that are NaN are never selected.
 */
size_t q4_lmhead_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K);
q4_status q4_lmhead_argmax(const void* w_q4, const float* x,
                           int32_t* out_idx, float* out_val,
                           int64_t M, int64_t N, int64_t K,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * q4_decode_chain -- one greedy decode step's Q4_0 work as one call (section
 * "Architecture": the decoder of width 3072 runs its projections once per
 * generated token, the LM head picks the token; section "Solutions
 * techniques pour l'exécution dans le navigateur", item 3: the 131072-row
 * table in Q4 gives both the logits and the next token's embedding).
 *   steps[0 .. nsteps-1] : matvecs run in order at M = 1,
 *                          y[n] = sum_k deq(W)[n, k] x[k]; a step starts
 *                          reading its x only after every earlier step has
 *                          written its y, so x may lie inside an earlier y.
 *                          The array is read during the call only.
 *   table_q4 (nullable)  : the tied table, vocab rows of dim.  If given, the
 *                          argmax over deq(T) head_x follows the steps
 *                          (head_x may lie inside a step's y): out_idx[0]
 *                          = the lowest index of the maximum, out_val[0]
 *                          (nullable) the maximum, and out_embed (nullable,
 *                          dim floats) = deq(T[out_idx[0]]) -- the next
 *                          step's input, decoded by the argmax's last
 *                          workgroup in the same launch (zeros if no logit
 *                          is a number).
 *   workspace, ws_bytes  : as for q4_lmhead_argmax with M = 1 (256 bytes,
 *                          zero before the first call, left zero); needed
 *                          only with a table.
 *   0 <= nsteps <= Q4_CHAIN_MAX_STEPS; nsteps == 0 needs a table.
 * Same arithmetic and bounds as q4_matvec and q4_lmhead_argmax; every
 * argument is validated before anything is enqueued.  One launch per step
 * and one for the argmax and embedding, all on `stream`: on this chip a
 * kernel boundary (~2 us) orders the steps at less cost than a grid-wide
 * barrier inside one persistent kernel (measured 3.8 us with relaxed
 * atomics over 256 workgroups, 7.3 us with the release and acquire that the
 * memory model requires for the step's outputs to be visible).
 */
#define Q4_CHAIN_MAX_STEPS 64
typedef struct q4_matvec_step {
  const void* w_q4;  /* N rows of Q4_0, N*18*K/32 bytes (device)           */
  const float* x;    /* K floats (device)                                  */
  float* y;          /* N floats (device), written                         */
  int64_t N;
  int64_t K;
} q4_matvec_step;
q4_status q4_decode_chain(const q4_matvec_step* steps, int64_t nsteps, const void* table_q4,
                          int64_t vocab, int64_t dim, const float* head_x, int32_t* out_idx,
                          float* out_val, float* out_embed, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * q4_lmhead_argmax_noalloc -- q4_lmhead_argmax for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * q4_lmhead_argmax without the workspace: its place is taken by a fixed
 * 16 KiB array in the library's own device memory (one per GPU, held until
 * the process ends), so 1 <= M <= 64 (Q4_ERR_SHAPE beyond).  Allocates
 * nothing.  The first call on a device also enqueues one small kernel that
 * clears that array.  Every call on one GPU shares the array, so calls that
 * may overlap on one GPU (unordered streams) race: the caller orders them.
 */
q4_status q4_lmhead_argmax_noalloc(const void* w_q4, const float* x, int32_t* out_idx,
                                   float* out_val, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Diagnostics: which kernel a call takes (the tests use these to cover every
 * kernel; a caller may log them).  Both return a static string, or NULL for
 * a shape the entry point rejects; they enqueue nothing.
 * q4_matmul_route: the kernel q4_matmul runs for (M, N, K) with a workspace
 *   of ws_bytes on the current device -- "matvec" (the q4_matvec kernel,
 *   rows of x in pairs), "small" (M <= 4, weights read once), "stream16"
 *   (3 to 16 rows with K <= 6144, up to 48 rows with K <= 3072, two rows
 *   with K <= 3072 over 20 MiB of weights: tiles of 16 rows of x, weights
 *   read once), "skinny" (the other prompt-prefix
 *   shapes up to 48 rows), "wide128" / "wide96" /
 *   "wide64" / "wide32" (tiles of 128, 96, 64 or 32 rows of X by 256
 *   outputs), "tile" (128 x 128, narrow outputs) or "simple" (K % 64 == 32)
 *   -- and, if splits is not NULL, its number of K splits (1: none).
 * q4_matvec_route: the kernel variant q4_matvec (argmax == 0) or
 *   q4_lmhead_argmax (argmax != 0) runs for an N x K matrix -- "pairs_lds_g4"
 *   (x in LDS, four row groups per workgroup: 65536 rows or more),
 *   "pairs_lds" (x in LDS), "pairs_reg_r1" / "pairs_reg_r2" (x in registers,
 *   one or two rows per lane and pass) or "any" (K % 64 == 32, or K > 12288).
 */
const char* q4_matmul_route(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int32_t* splits);
const char* q4_matvec_route(int64_t N, int64_t K, int32_t argmax);

/*
 * q4_quantize -- device-side GGUF Q4_0 encoder, used to prepare weights:
 * per block of 32 values, m = the first element of largest magnitude,
 * d = m / -8 in float32 stored as binary16 (round to nearest even), codes
 * q = clamp(floor(x / d + 1/2) + 8, 0, 15) decided in float64 against the
 * stored scale (q = 8 everywhere when it is zero).
 *   w     : [N, K] float32.   w_q4 : N*18*K/32 bytes (written).
 *   flag  : device int32 or NULL; set to 1 (never cleared) if any input is
 *           not finite or a scale overflows binary16 -- the bytes of such a
 *           block are then unspecified.
 */
q4_status q4_quantize(const float* w, void* w_q4, int64_t N, int64_t K,
                      int32_t* flag, void* stream);

/*
 * GGUF reader (host code, no GPU) -- the container of the pages' quantised
 * model (section "Architecture": a GGUF Q4_0 file; section "Préparation du
 * modèle et sharding": the file is cut into byte pieces of at most 512 MB).
 *
 * q4_gguf_open: paths[0 .. npaths-1] are read as ONE byte stream, in order
 * (one file, or the pieces of a byte-level split).  Parses the header
 * ("GGUF", version 2 or 3), the metadata, the tensor table and the alignment
 * ("general.alignment", default 32), and checks that every tensor of a known
 * element type lies inside the data section.  On success *out owns open file
 * descriptors until q4_gguf_close.  Errors: Q4_ERR_NULL, Q4_ERR_IO (open or
 * read failed), Q4_ERR_FORMAT (bad magic or version, truncated or
 * inconsistent tables, duplicate tensor names, misaligned offsets).
 *
 * Tensors: dims[0] is the innermost dimension (a weight of N rows of K is
 * dims = {K, N, 1, 1}).  Element types sized here: 0 F32, 1 F16, 2 Q4_0,
 * 8 Q8_0, 30 BF16; other types are listed with nbytes = 0 and cannot be read.
 * A Q4_0 tensor's bytes are exactly the layout q4_matvec / q4_matmul take.
 * q4_gguf_read_tensor copies a tensor into HOST memory dst (dst_bytes >=
 * nbytes, else Q4_ERR_WORKSPACE).  Metadata getters look a key up by name:
 * integers (any integer or bool type, as int64), floats (F32/F64 as double),
 * strings (pointer valid until close), arrays (element type and count only).
 * Returned name/key/string pointers are owned by the handle.  A handle may be
 * read from several threads at once (pread); open/close are not concurrent
 * with its use.
 */
typedef struct q4_gguf q4_gguf;
q4_status q4_gguf_open(const char* const* paths, int64_t npaths, q4_gguf** out);
void q4_gguf_close(q4_gguf* g);
uint32_t q4_gguf_version(const q4_gguf* g);
uint64_t q4_gguf_alignment(const q4_gguf* g);
uint64_t q4_gguf_data_offset(const q4_gguf* g);
int64_t q4_gguf_tensor_count(const q4_gguf* g);
int64_t q4_gguf_metadata_count(const q4_gguf* g);
q4_status q4_gguf_tensor_info(const q4_gguf* g, int64_t index, const char** name,
                              uint32_t* type, uint32_t* n_dims, int64_t* dims4,
                              uint64_t* offset, uint64_t* nbytes);
int64_t q4_gguf_find_tensor(const q4_gguf* g, const char* name);  /* -1: absent */
q4_status q4_gguf_read_tensor(const q4_gguf* g, int64_t index, void* dst,
                              uint64_t dst_bytes);
q4_status q4_gguf_metadata_key(const q4_gguf* g, int64_t index, const char** key,
                               uint32_t* value_type);
q4_status q4_gguf_metadata_int(const q4_gguf* g, const char* key, int64_t* value);
q4_status q4_gguf_metadata_float(const q4_gguf* g, const char* key, double* value);
q4_status q4_gguf_metadata_string(const q4_gguf* g, const char* key,
                                  const char** value, uint64_t* length);
q4_status q4_gguf_metadata_array(const q4_gguf* g, const char* key,
                                 uint32_t* elem_type, uint64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* Q4MI_Q4_H */
