/*
 * spec_verify.h - batched speculative-sampling verification on MI355X (gfx950).
 *
 * What is computed.  For each of B sequences the caller supplies draft logits
 * and target logits at gamma+1 positions over a V-token vocabulary, the gamma
 * draft tokens x_0..x_{gamma-1}, a temperature T and uniforms.  With
 * p_i = softmax(draft_i / T) and q_i = softmax(target_i / T):
 *
 *   - position i is accepted iff u_accept[b][i] < min(1, q_i(x_i) / p_i(x_i))
 *     ("Speculative Decoding: small model guesses, large model verifies",
 *      section 3: the acceptance rule; section 5.4: same T on both sides);
 *   - k = the first rejected position, or gamma if none (section 3: stop at
 *     the first rejection; section 2: 1..gamma+1 tokens per round);
 *   - if k < gamma a token y is drawn from the residual (q_k - p_k)+ / sum(q_k - p_k)+
 *     (section 3), or with spec_verify_saguaro from
 *     sqrt(p_k * max(r, eps)) / sum, r = the normalised residual
 *     ("Speculative Speculative Decoding (Saguaro)", section 3.2);
 *   - if k == gamma the bonus token y is drawn from q_gamma (section 2: the
 *     target scores gamma+1 positions);
 *   - every draw takes the first token id j whose running probability sum in
 *     token-id order exceeds u_sample[b][k] (section 3, the choice helper);
 *     a residual draw whose residual mass is below 1/16 of q_k's is taken
 *     in fp64 from the logits (a kernel after the call's others), so that
 *     its running sums stay within 1e-6 of the exact ones;
 *   - the committed length is in_len + k + 1 (SSD summary, AMD MI300X part:
 *     on rejection only the valid-length pointer of the KV cache moves).
 *
 * Conventions for every entry point.
 *   - All array pointers are DEVICE pointers; `stream` is a hipStream_t passed
 *     as void* (NULL = the default stream).  Calls only enqueue work on that
 *     stream and return; nothing is synchronised.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory; its only global state is a per-device cache of how many
 *     work-groups the GPU holds at once (queried on the first call; its
 *     entries are atomics, so host threads may call concurrently).
 *     Concurrent calls need distinct workspaces.
 *   - Logits are row-major [B][gamma+1][V], contiguous, float32 (SPEC_F32) or
 *     bfloat16 (SPEC_BF16).  Row i of sequence b starts at element
 *     (b*(gamma+1)+i)*V.  The verification reads draft rows 0..gamma-1 and
 *     target rows 0..gamma; draft row gamma is read only by outcome prediction.
 *   - Host-checkable errors return a negative status before anything is
 *     enqueued: B < 0, gamma outside [1, 63], V < 1 or V > 2^30,
 *     B * (2 gamma + 1) * ceil(V / 2048) > 2^29 (about 2^40 logits per tensor,
 *     beyond any one GPU's memory; it keeps every count in 32 bits), T not
 *     finite or <= 0,
 *     eps not finite or < 0, a NULL required pointer, an unknown dtype, a
 *     workspace smaller than spec_workspace_bytes().  B == 0 is a no-op.
 *   - Data errors found on the device mark only their sequence: a draft token
 *     outside [0, V), or a row read by the rule that holds a NaN or +inf
 *     logit (or only -inf logits).  Such a sequence gets accepted = -1, every
 *     token -1, first_reject = -1, mask = 0, out_len = in_len.
 *   - A launch failure returns SPEC_ELAUNCH.  No exception crosses the ABI.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum spec_status {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,     /* bad size, temperature, eps or NULL pointer */
  SPEC_EDTYPE = -2,     /* dtype is neither SPEC_F32 nor SPEC_BF16 */
  SPEC_EWORKSPACE = -3, /* workspace NULL or smaller than required */
  SPEC_ELAUNCH = -4,    /* a kernel launch failed */
  SPEC_ESCRATCH = -5    /* spec_verify_noalloc: the sizes need more than its static scratch */
};

enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 };

/*
 * Optional diagnostics (pass NULL in production).  Each field is an optional
 * device pointer; NULL fields are skipped.  Values are those the device used.
 *   row_max, row_logZ: [B][2*gamma+1], draft rows 0..gamma-1 then target rows
 *     0..gamma: max_j l_j / T and log sum_j exp(l_j / T).
 *   px, qx: [B][gamma] p_i(x_i), q_i(x_i).
 *   resid_mass: [B] sum_j (q_k - p_k)+ (0 when k == gamma).
 *   token_prob: [B] probability of y under the distribution it was drawn from.
 *   cdf_lo, cdf_hi: [B] the running sums C_{y-1} and C_y of that distribution.
 * Invalid sequences leave their entries unwritten.
 */
typedef struct spec_diag {
  double* row_max;
  double* row_logZ;
  double* px;
  double* qx;
  double* resid_mass;
  double* token_prob;
  double* cdf_lo;
  double* cdf_hi;
} spec_diag;

/*
 * Bytes of device workspace spec_verify / spec_verify_saguaro need for these
 * sizes (0 when B == 0).  Returns 0 for arguments spec_verify would reject.
 * The workspace must be zero-filled before its first use; each call that
 * completes leaves it ready for the next one, so a workspace is allocated and
 * cleared once and then reused by calls on one stream.  Its first 32-bit word
 * is an error flag: the kernels hand partial results between work-groups
 * through the workspace and wait for them with bounded polls.  A poll that
 * times out (never expected) sets the word to 1; from then on every wait of
 * the call gives up within a few microseconds, every kernel returns, and no
 * sequence is reported valid from a value that did not arrive: a sequence
 * whose decision is taken with the word set, or any of whose waits gave up,
 * comes back invalid (accepted = -1, tokens -1).  The call still returns
 * SPEC_OK (nothing is synchronised); check the word after the stream, and
 * zero the whole workspace before reusing it once it is set.  The second
 * 32-bit word is the check word of the library's checks build (a separate
 * library, compiled with SV_CHECKS=1, that tests every index its kernels form
 * against the size of its array): nonzero names the site of the first failed
 * test, whose index was clamped into range.  The default build never writes
 * it.  spec_verify_greedy's workspace starts the same way.
 */
size_t spec_workspace_bytes(int B, int gamma, int V, int dtype);

/*
 * Verification with residual resampling.
 *   draft_logits, target_logits: [B][gamma+1][V] of `dtype`.
 *   draft_tokens: [B][gamma] int32.
 *   u_accept: [B][gamma] float, u_sample: [B][gamma+1] float, values in [0, 1).
 *   temperature: T > 0, applied to both models.
 *   in_len: [B] int32 committed lengths before the round; NULL = zeros.
 * Outputs ([B] unless stated):
 *   out_tokens: [B][gamma+1] int32: x_0..x_{k-1}, y, then -1.
 *   out_accepted: k (number of accepted draft tokens).
 *   out_first_reject: k if k < gamma else -1 (nullable).
 *   out_accept_mask: bit i = decision at position i for all i < gamma (nullable).
 *   out_len: in_len + k + 1 (nullable).
 *   diag: NULL or a host pointer to a spec_diag of optional device pointers.
 */
int spec_verify(const void* draft_logits, const void* target_logits, int dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                int B, int gamma, int V, float temperature, const int32_t* in_len,
                int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * As spec_verify, but a rejection at k draws from the Saguaro distribution
 * proportional to sqrt(p_k(j) * max(r_j, eps)), r = (q_k - p_k)+ / sum(q_k - p_k)+
 * ("Speculative Speculative Decoding (Saguaro)", section 3.2).  eps = 0 is the
 * section's formula; eps = 1e-8 reproduces the clamp in its code.  The bonus
 * draw (k == gamma) is unchanged.
 */
int spec_verify_saguaro(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept,
                        const float* u_sample, int B, int gamma, int V, float temperature,
                        const int32_t* in_len, int32_t* out_tokens, int32_t* out_accepted,
                        int32_t* out_first_reject, uint64_t* out_accept_mask, int32_t* out_len,
                        const spec_diag* diag, void* workspace, size_t workspace_bytes,
                        void* stream, float eps);

/*
 * Bytes of device workspace spec_predict_outcomes needs (same zero-on-entry
 * rule as spec_workspace_bytes).
 */
size_t spec_predict_workspace_bytes(int B, int gamma, int V, int dtype);

/*
 * Outcome prediction for speculative speculative decoding
 * ("Speculative Speculative Decoding (Saguaro)", section 3.1: an outcome is
 * (k accepted, bonus token); the bonus is predicted from the draft logits'
 * top-3).  For every sequence b and every k in 0..gamma, cand[b][k][0..2]
 * are the token ids of the three largest draft logits at position k,
 * descending, equal logits ordered by lower id (+0.0 and -0.0 are equal); a
 * row holding a NaN gives -1 candidates.  3*(gamma+1) candidates per sequence.
 *   draft_logits: [B][gamma+1][V] of dtype (all gamma+1 rows are read).
 *   accepted, out_tokens: a verification's out_accepted [B] and out_tokens
 *     [B][gamma+1], or both NULL to compute candidates only.
 *   cand: [B][gamma+1][3] int32.
 *   hit: [B] int32 (nullable): 1 iff out_tokens[b][k] is one of cand[b][k],
 *     k = accepted[b]; 0 for an invalid sequence (accepted < 0).
 *   cand_idx: [B] int32 (nullable): 3k + rank of the matching candidate, or -1.
 */
int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int gamma, int V,
                          const int32_t* accepted, const int32_t* out_tokens, int32_t* cand,
                          int32_t* hit, int32_t* cand_idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Verification and outcome prediction in one pass over the logits
 * ("Speculative Speculative Decoding (Saguaro)", section 3.1: the outcomes
 * (k, bonus) are enumerated from the draft logits' top-3 and checked against
 * the verification's result).  The verification arguments and outputs are
 * those of spec_verify (saguaro = 0; eps is ignored) or spec_verify_saguaro
 * (saguaro = 1, eps as there); any other saguaro value is SPEC_EINVAL.  The
 * outcome outputs are those of spec_predict_outcomes given this call's
 * out_accepted and out_tokens:
 *   cand: [B][gamma+1][3] int32 (required); hit, cand_idx: [B] int32 (nullable).
 * The draft rows are read once: while the verification streams draft rows
 * 0..gamma-1 it also ranks them, and it streams draft row gamma for the
 * ranking alone.  The workspace is the verification's (spec_workspace_bytes),
 * with the same zero-on-entry rule; outputs equal those of the two separate
 * calls.
 */
int spec_verify_predict(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        int saguaro, float eps, int32_t* cand, int32_t* hit, int32_t* cand_idx,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Early-exit verification: the rule's loop with its break, reading a
 * position's rows only while every earlier position was accepted
 * ("Speculative Decoding: small model guesses, large model verifies",
 * section 3: test position i, stop at the first rejection).  Arguments,
 * workspace and outputs as spec_verify (saguaro = 0; eps ignored) or
 * spec_verify_saguaro (saguaro = 1); any other saguaro value is SPEC_EINVAL.
 * The tokens, k, first_reject and out_len equal spec_verify's; what differs:
 *   - out_accept_mask holds the decisions the loop makes: bits 0..k-1 (all
 *     set), never a decision after the first rejection;
 *   - validity only concerns what the loop reads: draft tokens x_0..x_k
 *     (x_0..x_{gamma-1} when k == gamma), draft and target rows 0..k (k <
 *     gamma), target row gamma only when k == gamma;
 *   - diagnostics exist only for the rows and positions read (other entries
 *     are left unwritten).
 * Positions are processed in order across the whole batch, and a rejection
 * is published as soon as it is known, so the rows of later positions of
 * that sequence are usually not read at all (how many are skipped depends on
 * timing; the outputs do not).
 */
int spec_verify_early(const void* draft_logits, const void* target_logits, int dtype,
                      const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                      int B, int gamma, int V, float temperature, const int32_t* in_len,
                      int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                      uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                      int saguaro, float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Options of spec_verify_ex.  A zero-filled struct (or a NULL pointer) is
 * spec_verify's behaviour.
 *   saguaro, eps: as spec_verify_saguaro when saguaro == 1 (0: residual).
 *   early: nonzero = early exit, as spec_verify_early.
 *   temperature: NULL, or a DEVICE array [B] of per-sequence temperatures
 *     that replaces the scalar argument (which is then not checked): sequence
 *     b uses T_b for both models ("Speculative Decoding: small model guesses,
 *     large model verifies", section 5.4: the same temperature on both sides;
 *     section 3, after its numerical check of unbiasedness: the rule stacks on
 *     temperature sampling unchanged).
 *     A T_b that is not finite and positive makes only that sequence invalid.
 *   cand, hit, cand_idx: outcome prediction outputs as spec_verify_predict
 *     (cand NULL = no prediction; hit / cand_idx need cand).
 *   top_p: 0 or 1 = no cut; in (0, 1): every row's distribution (draft rows
 *     0..gamma-1, target rows 0..gamma) is cut to its nucleus and
 *     renormalised, and the rule runs on the cut distributions (same section
 *     3 remark: the rule stacks on top-p sampling; section 5.4: the same
 *     setting on both sides).  The nucleus is every token whose logit is >= L,
 *     L the largest logit value at which the mass of the tokens with logits
 *     >= L reaches top_p (equal logits all in or all out).  Diagnostics report
 *     p(x), q(x), pi(y) and the running sums of the cut distributions and the
 *     row statistics of the uncut rows.  Outside [0, 1] or NaN: SPEC_EINVAL.
 * early combines with neither prediction nor a top-p cut (SPEC_EINVAL).
 */
typedef struct spec_options {
  int saguaro;
  float eps;
  int early;
  const float* temperature;
  int32_t* cand;
  int32_t* hit;
  int32_t* cand_idx;
  float top_p;
} spec_options;

/*
 * Verification with options: the arguments of spec_verify plus `opts` (a
 * host pointer, may be NULL).  Workspace: spec_workspace_bytes().
 */
int spec_verify_ex(const void* draft_logits, const void* target_logits, int dtype,
                   const int32_t* draft_tokens, const float* u_accept, const float* u_sample, int B,
                   int gamma, int V, float temperature, const int32_t* in_len, int32_t* out_tokens,
                   int32_t* out_accepted, int32_t* out_first_reject, uint64_t* out_accept_mask,
                   int32_t* out_len, const spec_diag* diag, const spec_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace spec_verify_greedy needs (same zero-on-entry rule
 * and error word as spec_workspace_bytes; 0 for B == 0 or arguments
 * spec_verify_greedy would reject).
 */
size_t spec_greedy_workspace_bytes(int B, int gamma, int V, int dtype);

/*
 * Greedy verification: the temperature -> 0 limit of the rule
 * ("Speculative Decoding: small model guesses, large model verifies",
 * sections 3 and 5.4; greedy and sampling modes as in "SSSD: Simply-Scalable
 * Speculative Decoding", training-strategy section).  With g_i the lowest
 * token id among the largest logits of target row i:
 *   - position i is accepted iff draft_tokens[b][i] == g_i (all gamma
 *     decisions are reported in the mask);
 *   - k = the first rejected position, or gamma;
 *   - the emitted token is g_k (the correction after a rejection, the bonus
 *     from row gamma after gamma acceptances).
 * Only target rows are read (no draft logits, no uniforms, no temperature).
 *   target_logits: [B][gamma+1][V] of dtype; draft_tokens: [B][gamma] int32.
 *   in_len and the outputs are as in spec_verify.
 * A sequence is invalid (accepted = -1, tokens -1, first_reject -1, mask 0,
 * out_len = in_len) when a draft token lies outside [0, V) or a row the rule
 * reads holds a NaN: rows 0..gamma-1 always, row gamma iff k == gamma.
 * Infinite logits are ordinary values here.  Host-checkable errors as for
 * spec_verify; the workspace is spec_greedy_workspace_bytes() bytes.
 */
int spec_verify_greedy(const void* target_logits, int dtype, const int32_t* draft_tokens, int B,
                       int gamma, int V, const int32_t* in_len, int32_t* out_tokens,
                       int32_t* out_accepted, int32_t* out_first_reject,
                       uint64_t* out_accept_mask, int32_t* out_len, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * A timed stand-in for a model forward pass, for scheduling experiments
 * around the verification ("Speculative Speculative Decoding (Saguaro)",
 * section 4.1: the draft model runs on its own stream while the target
 * verifies; SSD summary, AMD MI300X part: two HIP streams and events).  It
 * keeps one work-group of `stream` busy for `ns` nanoseconds of wall time
 * (0 <= ns <= 1e8), so it occupies its stream without taking the compute
 * units the verification uses.  With hit != NULL (a DEVICE array [n] of a
 * prediction's hit flags) it first checks them on the device and returns at
 * once when none is 0 (no fallback pass is needed).  Enqueues only.
 */
int spec_synthetic_busy(int64_t ns, const int32_t* hit, int n, void* stream);

/*
 * Synthetic bigram models for the pipeline of "Speculative Speculative
 * Decoding (Saguaro)", sections 3.1 and 4.1 (no weights exist here).  A model
 * is a DEVICE table [H][V] (dtype SPEC_F32 or SPEC_BF16, row-major, H >= 1;
 * H = V gives every token its own row): after token t its logits are row
 * t mod H.  Draft sampling is the Gumbel-max form: the token drawn at
 * absolute position pos after token t is
 *     argmax_j ( float(table[t mod H][j]) + noise[pos mod P][j] )
 * with one fp32 addition per candidate and ties to the lower id; `noise` is a
 * DEVICE float array [P][V] of T-scaled Gumbel variates (argmax_j(l_j/T + g_j)
 * with standard Gumbel g is a draw from softmax(l/T)), P >= 1.  1 <= gamma <= 63.
 * The caller owns every buffer; the calls enqueue on `stream` and return
 * SPEC_EINVAL for a NULL required pointer or a size out of range, SPEC_ELAUNCH
 * for a failed launch.  A token outside [0, V) where one is read makes the
 * tokens drawn from it -1 and the rows that follow it NaN (so the verification
 * marks the sequence invalid, and it stays so).
 *
 * spec_synth_draft: n chains of gamma draft steps; chain c starts after token
 *   start_tok[c] at position start_pos[c] (NULL: 0) and writes out_tokens[c][i],
 *   the token at position start_pos[c] + i.
 * spec_synth_rows: a round's logits [B][gamma+1][V] (dtype of the table): row i
 *   of sequence b is the table row (mod H) of the token before position i, which is
 *   last[b] for i = 0 and tokens[b][i-1] ([B][gamma]) after.
 * spec_ssd_prespeculate: the next round's drafts for every predicted outcome,
 *   while the current round verifies.  cand [B][gamma+1][3] holds the draft's
 *   top-3 at each position (spec_predict_outcomes); outcome c = 3k + rank is
 *   "k drafts accepted, then cand[b][k][rank]", which leaves the sequence at
 *   length len[b] + k + 1 (len [B], NULL: 0) with that token last, and
 *   prepared[b][c][0..gamma) ([B][3(gamma+1)][gamma]) receives the drafts
 *   that follow it.
 * spec_ssd_advance: after a round's verification (out_tokens [B][gamma+1],
 *   accepted [B], out_len [B], all from spec_verify*): next_last[b] = the
 *   emitted token y (out_tokens[b][accepted[b]]), next_len[b] = out_len[b], and
 *   next_tokens[b] ([B][gamma]) the drafts that follow y: prepared[b][cand_idx[b]]
 *   when hit[b] != 0 (a hit of the prediction, spec_verify_predict), drawn
 *   after the verification otherwise (hit == NULL: always).  A sequence with
 *   accepted[b] < 0 gets next_last -1 and drafts -1.
 */
int spec_synth_draft(const void* table, int dtype, int V, int H, const float* noise, int P,
                     int gamma, int n, const int32_t* start_tok, const int32_t* start_pos,
                     int32_t* out_tokens, void* stream);
int spec_synth_rows(const void* table, int dtype, int V, int H, int gamma, int B,
                    const int32_t* last, const int32_t* tokens, void* out_rows, void* stream);
int spec_ssd_prespeculate(const void* table, int dtype, int V, int H, const float* noise,
                          int P, int gamma, int B, const int32_t* cand, const int32_t* len,
                          int32_t* prepared, void* stream);
int spec_ssd_advance(const void* table, int dtype, int V, int H, const float* noise, int P,
                     int gamma, int B, const int32_t* out_tokens, const int32_t* accepted,
                     const int32_t* out_len, const int32_t* hit, const int32_t* cand_idx,
                     const int32_t* prepared, int32_t* next_last, int32_t* next_len,
                     int32_t* next_tokens, void* stream);

/*
 * spec_verify without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing.  Its workspace is a static
 * array of 16 MiB in the library's device memory, one per GPU (held until the
 * process ends), which the call clears with a kernel before it runs.  Arguments,
 * outputs and results are those of spec_verify; sizes whose workspace
 * (spec_workspace_bytes) exceeds 16 MiB - at gamma = 8, V = 152064 in bf16,
 * B above 400 - return SPEC_ESCRATCH before anything is enqueued.  Every call
 * on one GPU shares that array: calls that overlap on one GPU (different
 * streams, or host threads) race and give undefined results; serialise them.
 * The array keeps the last call's contents, including a set error word (see
 * spec_workspace_bytes), which the next call clears.
 */
int spec_verify_noalloc(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        void* stream);

/*
 * A measurement aid, not part of the verification: reads `bytes` bytes of the
 * device buffer `buf` with the loads the verification's stream items use
 * (16-byte nontemporal loads, 64 KB per work-group), so that the HBM read
 * bandwidth attainable for a pass over the same bytes can be set beside the
 * verification's own rate.  `sink` is a device word written only if the
 * combined data equals an impossible value (it keeps the loads).  bytes must
 * be a positive multiple of 16 and buf 16-byte aligned, else SPEC_EINVAL.
 * Enqueues only.
 */
int spec_read_bandwidth(const void* buf, size_t bytes, uint64_t* sink, void* stream);

/*
 * A measurement aid, not part of the verification: the cost of an LDS atomic
 * add by how a wave's lanes fall on words and banks, which the top-p
 * counting kernel's counter layout is designed around.  One 1024-thread
 * work-group per CU; each wave adds 1 to words of its own 2048-word region,
 * 8 x iters wave-wide adds, lane l to word: pattern 0: l (64 words, 64
 * banks); 1: l / 8 (8 words, 8 lanes each); 2: 0 (one word); 3: 64 (l mod 32)
 * (32 words on one bank).  The caller times the launch on `stream`.  `sink`
 * is a device word written only if a count equals an impossible value.
 * pattern outside 0..3, iters outside 1..2^20 or a null sink: SPEC_EINVAL.
 * Enqueues only.
 */
int spec_lds_atomic_probe(int pattern, int iters, uint64_t* sink, void* stream);

/* A static, human-readable description of a status code. */
const char* spec_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
