/*
 * spec_verify.h - C ABI of the one-round draft-token verification library
 * (libspecverify.so, HIP for AMD Instinct MI355X / gfx950).
 *
 * The operation is the verification step of one speculative-decoding round as
 * defined in chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash, DDTree,
 * and DSpark", section 1, and the vLLM blog post "speculative-decoding-amd-gpus",
 * section "Core idea of speculative decoding":
 *
 *   - drafts are checked left to right and the round is cut at the first
 *     rejection; later drafts are discarded;
 *   - stochastic requests keep draft y_i with probability min(1, p_i(y_i)/q_i(y_i)),
 *     p_i = softmax(target logits / T), q_i = softmax(draft logits / T); at the
 *     first rejection the correction is drawn from the normalised residual
 *     [p_i - q_i]_+; if every draft survives a bonus token is drawn from the
 *     target row that follows the last draft;
 *   - greedy requests keep a draft while it equals the target argmax (lowest id
 *     on ties) and commit the target's argmax at the first mismatch, or the
 *     argmax of the bonus row when every draft survives.
 *
 * Randomness is supplied by the caller: one uniform u_i in [0,1) per draft
 * position (keep iff u_i * q(y_i) < p(y_i)) and one uniform w_b in [0,1) per
 * request for the single final draw, which takes the first token id t (in
 * ascending id order) whose running sum of weights exceeds w_b times their
 * total.  With the same inputs every call returns the same bits.
 *
 * Packed ragged layout.  Request b has k_b = num_draft[b] >= 0 drafts.  With
 * off[b] = k_0 + ... + k_{b-1} and K = off[B]:
 *   target row (b, i), i = 0..k_b  is row off[b] + b + i   (row k_b = bonus row)
 *   draft  row (b, i), i < k_b     is row off[b] + i, draft token draft_tokens[off[b]+i]
 *   out_tokens slot (b, i), i = 0..k_b is out_tokens[off[b] + b + i]
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library allocates nothing and keeps no state between
 *     calls (apart from the static device array that spec_verify_sample_noalloc
 *     uses in place of a workspace); calls are asynchronous on `stream` (a
 *     hipStream_t, NULL = the default stream) and results are valid once the
 *     stream reaches the call.
 *     Outputs must not overlap the inputs, each other or the workspace; two
 *     calls in flight at once need two workspaces.
 *   - Host-side argument checks run before any HIP call.  A failed check
 *     returns an error status and launches nothing and writes nothing.
 *   - SV_ERR_HIP reports a failed kernel launch (hipGetLastError).
 *   - Device-side input problems are reported in the outputs, never by a
 *     fault: if sum(num_draft) != K or some num_draft[b] < 0, every
 *     accepted_len is -1 and every output slot is -1; a stochastic request
 *     whose draft token lies outside [0, V) gets accepted_len -1, all its
 *     slots -1 and p_draft, q_draft, resid_mass -1.  Greedy requests compare
 *     such a token like any other id.
 *   - Logits must be finite or -inf.  A stochastic request that tests a row
 *     (target or draft) whose logits are all -inf is reported like one with
 *     an invalid token; rows after its cut are not looked at.  NaN / +inf
 *     give unspecified (but in-range or -1) results.
 *   - Temperature: the fp32 arithmetic uses the one scale c = fl(log2(e)/T),
 *     i.e. softmax(z / T') with T' = log2(e)/c within a relative 2^-24 of T;
 *     p(y), q(y) and the ratio tests are evaluated in fp64 from fp32 row sums.
 *   - The final draw equals the exact draw (at temperature T) unless the
 *     exact crossing of w_b * total lies within 1e-6 of the total from an edge
 *     of the chosen id's cumulative interval: draws from p and from residuals
 *     whose total is at least 1/8 are made with fp32 weights (cumulative
 *     error about 1e-8, below 1e-7 of the mass), smaller residuals are redone
 *     in fp64 from the logits unless the fp32 crossing lies clear of both
 *     edges.
 *   - Unused out_tokens slots (after the committed a_b + 1 tokens) are -1.
 *   - No C++ exception crosses this interface.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad temperature, misalignment */
  SV_ERR_UNSUPPORTED = 2,  /* dtype not supported, or target/draft dtypes differ   */
  SV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required           */
  SV_ERR_HIP = 4           /* a HIP call or kernel launch failed                   */
} sv_status_t;

typedef enum {
  SV_F32 = 0,   /* IEEE binary32 logits                        */
  SV_BF16 = 1   /* bfloat16 logits (upper half of a binary32)  */
} sv_dtype_t;

/* One packed batch of requests (see the layout above). */
typedef struct sv_batch {
  int32_t B;                  /* number of requests, >= 1                          */
  int32_t K;                  /* total draft tokens, sum of num_draft, >= 0        */
  int32_t V;                  /* vocabulary size, 1 <= V <= 2^30                   */
  int32_t dtype;              /* sv_dtype_t of target and draft logits             */
  int64_t target_ld;          /* elements between consecutive target rows, >= V    */
  int64_t draft_ld;           /* elements between consecutive draft rows, >= V     */
  const int32_t* num_draft;   /* device [B]: k_b                                   */
  const void* target;         /* device [K+B][target_ld] logits                    */
  const void* draft;          /* device [K][draft_ld] logits; may be NULL for
                                 spec_verify_greedy                                */
  const int32_t* draft_tokens;/* device [K]; may be NULL when K == 0               */
} sv_batch_t;

/* Bytes of device workspace a call with these sizes needs (256-byte aligned
 * internally; any pointer alignment is accepted).  Returns 0 for invalid sizes. */
size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V);

/* Static, NUL-terminated description of a status code. */
const char* spec_verify_status_string(int32_t status);

/* Greedy verification of every request (chzhyang section 1, "Greedy
 * equivalence"; vLLM blog "A simple accept/reject example").  Reads target
 * rows only.  Outputs:
 *   accepted_len [B]  a_b = drafts kept (excludes the final target token)
 *   out_tokens [K+B]  slots (b, 0..a_b-1) = kept drafts, slot (b, a_b) = target
 *                     argmax of row (b, a_b), later slots -1.                  */
int32_t spec_verify_greedy(const sv_batch_t* batch,
                           int32_t* accepted_len, int32_t* out_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Stochastic verification (chzhyang section 1: acceptance probability
 * min(1, p/q), residual [p - q]_+ at the first rejection, bonus from the
 * target), optionally mixed with greedy requests.
 *   temperature   > 0 and finite, with log2(e)/temperature representable in
 *                 fp32 (temperature >= about 4.3e-39); applied to target and
 *                 draft logits alike.
 *   greedy_mask   device [B] or NULL; a non-zero byte makes request b greedy
 *                 (its draft rows, u_accept and u_final are then not read).
 *   u_accept      device [K] uniforms in [0,1), one per draft position.
 *   u_final       device [B] uniforms in [0,1), one per request.
 *   accepted_len, out_tokens  as for spec_verify_greedy; slot (b, a_b) holds
 *                 the correction or bonus draw.
 *   p_draft, q_draft  device [K] or NULL: p(y_i), q(y_i) of every draft row of
 *                 stochastic requests (also rows after the cut); -1 for greedy
 *                 requests.
 *   resid_mass    device [B] or NULL: total of [p - q]_+ at the cut (0 when it
 *                 is zero and the draw fell back to p), -1 when the bonus was
 *                 drawn or the request is greedy.                              */
int32_t spec_verify_sample(const sv_batch_t* batch, float temperature,
                           const uint8_t* greedy_mask,
                           const float* u_accept, const float* u_final,
                           int32_t* accepted_len, int32_t* out_tokens,
                           float* p_draft, float* q_draft, float* resid_mass,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Left-to-right verification with early exit (chzhyang section 1 and the vLLM
 * blog, "Core idea of speculative decoding": drafts after the first rejection
 * are discarded, so their rows need not be read).  Same results as
 * spec_verify_greedy / spec_verify_sample for accepted_len, out_tokens and
 * resid_mass, bit for bit, but reads the rows only up to a window past each
 * request's cut.  Round r verifies the positions [P_r, P_(r+1)) of every
 * request still alive, with P = 0, 1, 2, 4, 8, ... and the last window ending
 * at max_k + 1 (two kernel launches per round, plus one launch for the
 * residual sweeps of the last window's cuts); a request cut inside a window
 * has the rest of that window read but not used.
 *   max_k     bound on every num_draft[b], 0 <= max_k <= 4096; the call runs
 *             about log2(max_k) + 2 rounds.  A request with num_draft[b] >
 *             max_k is a device-side input error (every output -1, as for an
 *             inconsistent num_draft).
 *   p_draft, q_draft  p(y_i), q(y_i) of the positions actually tested (every
 *             position up to and including the cut); -1 for later positions,
 *             for greedy requests and for requests with an invalid token.
 * Other arguments, the workspace size and errors as for the functions above. */
int32_t spec_verify_greedy_early_exit(const sv_batch_t* batch, int32_t max_k,
                                      int32_t* accepted_len, int32_t* out_tokens,
                                      void* workspace, size_t workspace_bytes, void* stream);

int32_t spec_verify_sample_early_exit(const sv_batch_t* batch, int32_t max_k,
                                      float temperature, const uint8_t* greedy_mask,
                                      const float* u_accept, const float* u_final,
                                      int32_t* accepted_len, int32_t* out_tokens,
                                      float* p_draft, float* q_draft, float* resid_mass,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Acceptance statistics of verification outcomes, the signals of the vLLM blog
 * post "speculative-decoding-amd-gpus" ("Monitor acceptance behavior", and the
 * per-position columns of its Appendix tables).  Inputs are the accepted_len
 * [B] a call produced and the num_draft [B] it was given (device arrays);
 * rounds with accepted_len < 0 are not counted.  Writes device out[4 + max_pos]
 * (doubles):
 *   out[0] rounds counted n
 *   out[1] mean kept drafts  sum(a) / n                       (-1 if n == 0)
 *   out[2] MAL = 1 + out[1]: counts the correction/bonus token (-1 if n == 0)
 *   out[3] AR  = sum(a) / sum(k), kept over proposed drafts    (-1 if sum(k) == 0)
 *   out[3 + j], j = 1..max_pos: #{a >= j} / #{k >= j}         (-1 if no round
 *          proposed position j)
 * 1 <= max_pos <= 4096; host checks as for the other entry points.  One
 * workgroup; intended for batches of up to a few hundred thousand rounds. */
int32_t spec_verify_accept_stats(const int32_t* accepted_len, const int32_t* num_draft,
                                 int32_t B, int32_t max_pos, double* out, void* stream);

/* ---------------------------------------------------------------- token trees
 * Greedy verification of a draft token tree (chzhyang, "Speculative Decoding:
 * ...", section 5 "DDTree": the target scores every node with ancestor-only
 * attention; verification starts at the root and follows the child whose token
 * is the target's choice at the current node; when no child carries it, that
 * choice is the bonus token; only the walked path is kept).
 *
 * Packed layout.  Request b owns n_b = num_nodes[b] >= 1 nodes; with
 * noff[b] = n_0 + ... + n_{b-1} and N = noff[B], node i of request b is entry
 * noff[b] + i of parent / tokens and row noff[b] + i of target.  Node 0 is the
 * root (the last committed token; its token is not verified); every other
 * node i has a local parent index 0 <= parent < i.  Row i holds the target's
 * next-token logits after the prefix ending at node i.
 *
 * Greedy choice = lowest id attaining the row maximum.  If several children of
 * a node carry the chosen token, the lowest node index is followed.
 * Outputs (device, caller-owned):
 *   accepted_len [B]  a_b = draft nodes accepted (the root not counted)
 *   path_nodes   [N]  slots noff[b] + t, t = 0..a_b: local index of the t-th
 *                     node of the walk (t = 0: the root; its KV entries and
 *                     those of the listed nodes are the ones to keep)
 *   out_tokens   [N]  slots noff[b] + t, t < a_b: accepted tokens; slot
 *                     noff[b] + a_b: the bonus token
 *   every other slot -1.
 * Device-side input errors: if sum(num_nodes) != N or some num_nodes[b] < 1
 * every output is -1; a request with a parent outside [0, node) reports
 * accepted_len -1 and -1 slots.  Token values outside [0, V) are compared like
 * any id (they never match a choice).  Other conventions as above. */
typedef struct sv_tree {
  int32_t B;                  /* number of requests (trees), >= 1                   */
  int32_t N;                  /* total nodes, sum of num_nodes, >= B                */
  int32_t V;                  /* vocabulary size, 1 <= V <= 2^30                    */
  int32_t dtype;              /* sv_dtype_t of the target logits                    */
  int64_t target_ld;          /* elements between consecutive target rows, >= V     */
  const int32_t* num_nodes;   /* device [B]: n_b                                    */
  const int32_t* parent;      /* device [N]: local parent index (root's ignored)    */
  const int32_t* tokens;      /* device [N]: token of each node (root's ignored)    */
  const void* target;         /* device [N][target_ld] logits                       */
} sv_tree_t;

/* Workspace bytes for a tree call with these sizes (0 for invalid sizes). */
size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t N, int32_t V);

/* Reads every node row once, then walks each tree. */
int32_t spec_verify_tree_greedy(const sv_tree_t* tree, int32_t* accepted_len,
                                int32_t* path_nodes, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Same results, reading only the rows the walk can reach: round r takes the
 * steps [P_r, P_(r+1)) of every walk still going, P = 0, 1, 2, 4, 8, ... (two
 * kernel launches per round), after reading the row of each walk's current
 * node and of its descendants down to the window's last step (rows of
 * branches the walk does not take within the window are read but not used).
 * max_depth (0..4096) bounds a_b: the call runs about log2(max_depth) + 2
 * rounds, and a request whose walk would accept more than max_depth nodes is
 * an input error (accepted_len -1, -1 slots).  The tree depth is a safe bound. */
int32_t spec_verify_tree_greedy_early_exit(const sv_tree_t* tree, int32_t max_depth,
                                           int32_t* accepted_len, int32_t* path_nodes,
                                           int32_t* out_tokens, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- adaptive length
 * Confidence-driven verification length and compaction (chzhyang, "Speculative
 * Decoding: ...", section 5 DSpark: s_j = c_1 ... c_j estimates the chance of
 * accepting through position j and a window of k positions has estimated
 * progress 1 + s_1 + ... + s_k; section 2: the time per committed token is the
 * round's cost over its progress; section 9: the cost of each window length
 * comes from a table profiled for the deployment).
 *
 * Request b has a drafted block of N tokens (draft_tokens[b*N + i]) with
 * confidences conf[b*N + i] (fp32, used as given).  It keeps its first k_b
 * tokens, k_b in 0..N maximising (1 + s_1 + ... + s_k) / cost[k]; ties go to
 * the smallest k.  Arithmetic is fp64 in the order s = s * c_j,
 * total = total + s, ratio = total / cost[k] (correctly rounded), so the choice
 * is reproducible bit for bit.  Outputs (device, caller-owned):
 *   num_draft  [B]    k_b (the num_draft of the packed batch to verify)
 *   offsets    [B+1]  exclusive prefix sums of k_b; offsets[B] = K'
 *   tokens_out [B*N]  capacity; the first K' entries are the kept tokens,
 *                     request after request
 *   src_index  [B*N]  or NULL: b*N + i for each kept token (its row in the
 *                     drafter's [B*N] row layout, e.g. for
 *                     spec_verify_gather_rows)
 *   progress   [B]    or NULL: 1 + s_1 + ... + s_{k_b}
 * A cost table entry that is not a positive finite number is a device-side
 * input error: every num_draft and progress is -1, every offset 0, nothing is
 * compacted.  1 <= B, 0 <= N <= 4096.  One workgroup. */
int32_t spec_verify_adaptive_length(int32_t B, int32_t N, const float* conf,
                                    const double* cost, const int32_t* draft_tokens,
                                    int32_t* num_draft, int32_t* offsets,
                                    int32_t* tokens_out, int32_t* src_index,
                                    double* progress, void* stream);

/* Row gather for the compacted batch: dst row r = src row index[r] for
 * r < min(*count, max_rows) (count is a device pointer, e.g. &offsets[B] of
 * spec_verify_adaptive_length, so no host synchronisation is needed).  Rows
 * hold V elements of dtype; src_ld, dst_ld >= V are row strides in elements;
 * index has at least max_rows entries; a row whose index lies outside
 * [0, src_rows) is left unwritten.  An HBM-bound copy (nontemporal 16-byte
 * loads and stores when pointers and strides are 16-byte aligned). */
int32_t spec_verify_gather_rows(int32_t dtype, int32_t V, const void* src, int64_t src_ld,
                                int32_t src_rows, const int32_t* index, const int32_t* count,
                                int32_t max_rows, void* dst, int64_t dst_ld, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * spec_verify_sample with the same arguments and results, minus the workspace,
 * which is a static device array of SPEC_VERIFY_NOALLOC_MAX_BYTES that the
 * library holds on every device it runs on until the process ends.  The call
 * allocates nothing.  It runs the host checks of spec_verify_sample first, and
 * returns SV_ERR_WORKSPACE when spec_verify_workspace_bytes(B, K, V) exceeds
 * that size (for example B = 2048 requests with 8 drafts each at V = 262144
 * fit); a call refused either way makes no HIP call and writes nothing.  The
 * array's device address is looked up once per device, on the first call that
 * passes those checks (SV_ERR_HIP if that fails).  Every call
 * on one device uses the same array, which keeps the last call's contents:
 * calls that overlap on one device (two streams, two host threads) race and
 * must be serialised by the caller.  Launch plan and results as for
 * spec_verify_sample. */
#define SPEC_VERIFY_NOALLOC_MAX_BYTES (32u << 20)
int32_t spec_verify_sample_noalloc(const sv_batch_t* batch, float temperature,
                                   const uint8_t* greedy_mask,
                                   const float* u_accept, const float* u_final,
                                   int32_t* accepted_len, int32_t* out_tokens,
                                   float* p_draft, float* q_draft, float* resid_mass,
                                   void* stream);

/* Launch plan of spec_verify_greedy / spec_verify_sample for calls made from
 * the calling thread: 0 = automatic (default: one launch, one workgroup per
 * request, when the logit rows of the call total at most 48 MiB and B <= 2048;
 * otherwise the multi-kernel pipeline), 1 = always the multi-kernel pipeline,
 * 2 = always the single launch.  Both plans run the same arithmetic and return
 * the same bits.  Thread-local; SV_ERR_INVALID_ARG for other values. */
int32_t spec_verify_set_launch_plan(int32_t plan);

/* Diagnostic: a plain streaming read of `bytes` (a multiple of 16) at src
 * (16-byte aligned) with the access pattern of the row-statistics kernel (one
 * wavefront per 32 KiB unit, persistent grid, 16-byte nontemporal loads) and
 * no arithmetic on the data: the read bandwidth the streaming kernels are
 * measured against.  sink: device buffer of 64 uint32 that receives a store
 * only if the data folds to one fixed value.  Honours
 * spec_verify_set_profile_events. */
int32_t spec_verify_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Diagnostics for measurement tools.  When both are non-NULL (hipEvent_t
 * handles), later calls made from the calling thread record ev_begin just
 * before and ev_end just after the row-statistics kernel (for the early-exit
 * entry points: around all rounds), on the call's stream; tree calls too, and
 * spec_verify_gather_rows around its copy kernel.  Pass NULL, NULL to stop.  Thread-local; returns SV_OK. */
int32_t spec_verify_set_profile_events(void* ev_begin, void* ev_end);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
