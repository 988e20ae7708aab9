/*
 * sdkv.h -- C ABI of libsdkv: a dictionary-coded KV cache for AMD MI355X
 * (gfx950): greedy-pursuit encode and query-aware hierarchical decode
 * attention over coded keys and values.
 *
 * Method: "LLM Inference in a Flash!" (abstract page; review page, Summary,
 * Strengths and FAQ). Each key or value vector is stored as K (atom index,
 * coefficient) pairs over a static per-layer, per-stream dictionary of
 * unit-norm atoms (32,768 atoms, K = 16 on the pages). Decode scores every
 * cached token with its first Klow atoms, keeps the top fraction of tokens
 * and rescores those with Khigh atoms.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    row-major and densely packed in the layout stated per argument. The
 *    caller owns every buffer, including the workspace; the library never
 *    allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream and returns at once.
 *  - Code word: one uint32 per (index, coefficient) pair; bits 0-15 hold the
 *    atom index (uint16), bits 16-31 the IEEE binary16 coefficient.
 *  - Validation happens before anything is enqueued; on any error nothing
 *    is written. Kernel launch failures are reported as SDKV_ERR_DEVICE
 *    (faults inside an already-enqueued kernel surface at the caller's next
 *    synchronisation, as for any HIP kernel). No C++ exception crosses the
 *    ABI. Calls are reentrant and thread-safe on the host (the only
 *    process-wide state is a mutex-guarded cache of per-device kernel
 *    occupancy and the wait bounds of sdkv_test_set_wait); two calls that
 *    share a workspace must not overlap in time.
 *  - Co-residency. sdkv_decode_attn and sdkv_select_topk split long rows
 *    over several workgroups that wait for each other inside one launch
 *    (no cooperative launch). The host checks that the device can hold a
 *    row's workgroups at once, which assumes the call has the GPU to itself:
 *    concurrent work on other streams that occupies compute units (another
 *    of these calls, a persistent communication kernel) can leave a row's
 *    workgroups unable to meet. Such calls are unsupported. The waits are
 *    bounded (about half a second), so nothing hangs: a wait that gives up
 *    sets the workspace's status word (below) and the results of the call
 *    are then unreliable.
 *  - Status word. Word 0 (uint32) of the workspace of sdkv_decode_attn and
 *    sdkv_select_topk is cleared by the call and, once its work has
 *    completed on the stream, holds 0, or 1 if a cross-workgroup wait gave
 *    up (report it as SDKV_ERR_WAIT). Read it after synchronising.
 *  - Inputs must be finite. Code indices must be < n_atoms; other indices
 *    give unspecified (but in-bounds) results.
 *  - Dictionaries, encode inputs x, queries q and workspaces must start at
 *    16-byte aligned addresses (every torch allocation does), else
 *    SDKV_ERR_UNSUPPORTED; other pointers need their element's alignment.
 */
#ifndef SDKV_H
#define SDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SDKV_API __attribute__((visibility("default")))
#else
#define SDKV_API
#endif

#define SDKV_ABI_VERSION 8

typedef int32_t sdkv_status;
#define SDKV_OK 0
#define SDKV_ERR_NULL 1        /* a required pointer is NULL               */
#define SDKV_ERR_SHAPE 2       /* a size or count is out of range          */
#define SDKV_ERR_DTYPE 3       /* unknown dtype code                       */
#define SDKV_ERR_UNSUPPORTED 4 /* valid, but outside what the kernels take */
#define SDKV_ERR_WORKSPACE 5   /* workspace smaller than the query result  */
#define SDKV_ERR_DEVICE 6      /* a HIP runtime call or launch failed      */
#define SDKV_ERR_WAIT 7        /* (status word) a cross-workgroup wait gave
                                  up; never returned by a call itself       */

/* dtype codes */
#define SDKV_BF16 0
#define SDKV_F32 1

/* ------------------------------------------------------------------------
 * Encode: greedy projection pursuit (review page, Summary and Strengths: a
 * greedy pursuit that projects onto one atom per step and, unlike OMP, never
 * re-solves a least-squares problem). For every input vector x:
 *     r = x;  for k < K:  a_k = argmax_a |<r, d_a>|  (lowest a on ties),
 *                          g_k = <r, d_{a_k}>,  r -= g_k d_{a_k}.
 * Atoms are expected to have unit norm (the coefficient is not divided by
 * |d|^2). g_k and the residual are fp32. For n > 64 vectors an fp16
 * matrix-core screen of all atoms is followed by an exact fp32
 * recomputation of every atom the screen cannot rule out (the screen's
 * error is bounded from its fp16 rounding and the largest atom norm), so
 * the pick is the argmax of the exact fp32 correlations. For n <= 64 (a decode step's new
 * tokens, which the cache appends as codes: review page, Strengths, on
 * write endurance) every correlation is computed to fp32 accuracy with the
 * atoms spread over the whole device (bf16 dictionaries: the residual split
 * exactly into three bf16 parts on the matrix cores, products exact, fp32
 * accumulation; fp32 dictionaries: fp32 dot products); that path takes
 * K + 1 launches.
 * ---------------------------------------------------------------------- */
typedef struct sdkv_encode_args {
  const void* x;        /* [n, d] vectors, dtype x_dtype (SDKV_BF16/F32)  */
  int32_t x_dtype;
  const void* dict;     /* [n_atoms, d] atoms, dtype dict_dtype           */
  int32_t dict_dtype;
  int64_t n;            /* number of vectors, >= 1                        */
  int32_t d;            /* 64 or 128                                      */
  int32_t n_atoms;      /* 1 .. 65536                                     */
  int32_t K;            /* code length, 1 .. 32                           */
  uint32_t* codes;      /* OUT code words of vector i at codes[i * codes_ld
                           + k], k < K, pursuit order; required           */
  int64_t codes_ld;     /* words between vectors' code rows: 0 means K,
                           else >= K. Pointing `codes` at slot t of a
                           [rows, T, stride] cache with codes_ld = T *
                           stride appends one token per row in place.     */
  float* coef_f32;      /* OUT [n, K] unrounded g_k (OMP: the final
                           least-squares coefficients), or NULL           */
  float* resid_norm;    /* OUT [n] |r_K|_2, or NULL                       */
  uint32_t* low_plane;  /* OUT first klow code words of vector i at
                           low_plane[i * low_ld + j], or NULL             */
  int64_t low_ld;       /* 0 means klow, else >= klow                     */
  int32_t klow;         /* 1 .. K when low_plane != NULL                  */
  /* Optional stage timing: NULL, or SDKV_ENCODE_STAGES + 1 hipEvent_t
     handles (created by the caller); event i is recorded on `stream` before
     stage i and the last one after the final stage. Stages: 0 fp16 screen
     copy of the dictionary, 1 pursuit.                                   */
  void* const* stage_events;
  /* SDKV_ENCODE_PURSUIT (0): the greedy pursuit above. SDKV_ENCODE_OMP (1):
     orthogonal matching pursuit, the comparison encoder the pursuit
     replaces (review page, Summary and Strengths: the projection pursuit
     avoids OMP's least-squares refits): the same atom choice on the current
     residual, then every selected atom's coefficient refit by least squares
     and r = x - sum_j g_j d_{a_j}; the codes hold the final coefficients.
     Once the residual is exactly zero (a zero vector) every correlation is
     zero: the remaining slots take atom 0 with coefficient 0, as in the
     pursuit. Built as a comparison on the small path only: n <= 64 and bf16
     dictionaries, else SDKV_ERR_UNSUPPORTED; K + 2 launches. Other values:
     SDKV_ERR_SHAPE.                                                      */
  int32_t algorithm;
} sdkv_encode_args;
#define SDKV_ENCODE_PURSUIT 0
#define SDKV_ENCODE_OMP 1
#define SDKV_ENCODE_STAGES 2

/* Bytes of device workspace sdkv_encode needs for these arguments. */
SDKV_API sdkv_status sdkv_encode_workspace(const sdkv_encode_args* args, size_t* bytes);
SDKV_API sdkv_status sdkv_encode(const sdkv_encode_args* args, void* ws, size_t ws_bytes,
                        void* stream);

/* Two small encodes in one sequence of launches (K + 1; OMP: K + 2): a
 * decode step's new key vectors over the key dictionary and its value
 * vectors over the value dictionary (review page, Strengths, on write
 * endurance: a new token is appended as codes). Each side gets the codes,
 * coefficients, norms and low plane that sdkv_encode gives it alone, bit
 * for bit. Both must take the small path (n <= 64), else
 * SDKV_ERR_UNSUPPORTED, and agree in n, d, n_atoms, K, dict_dtype and
 * algorithm, else SDKV_ERR_SHAPE; stage_events are not recorded. The
 * workspace holds both sides' scratch; outputs must not overlap the inputs
 * or each other. */
SDKV_API sdkv_status sdkv_encode_pair_workspace(const sdkv_encode_args* key,
                                                const sdkv_encode_args* val, size_t* bytes);
SDKV_API sdkv_status sdkv_encode_pair(const sdkv_encode_args* key, const sdkv_encode_args* val,
                                      void* ws, size_t ws_bytes, void* stream);

/* sdkv_encode_pair without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the scratch lives in a static device array of
 * SDKV_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends, whose
 * address is looked up on the first call on each device. Same arguments,
 * kernels and results as sdkv_encode_pair (bit for bit); no allocation or
 * free. A problem whose scratch would exceed the array returns
 * SDKV_ERR_WORKSPACE (every n <= 64, n_atoms <= 65536, K <= 32 problem
 * fits). All calls on one GPU share its array, and the kernels write every
 * scratch word before reading it: calls that overlap in time on one GPU
 * (other streams, other host threads) race and are unsupported. */
#define SDKV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
SDKV_API sdkv_status sdkv_encode_pair_noalloc(const sdkv_encode_args* key,
                                              const sdkv_encode_args* val, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention for one layer and one decode step (review page, Summary:
 * every token gets a cheap score from its first Klow = 3 atoms and only the
 * best tenth is rescored with Khigh = 16; FAQ: three atoms suffice to score
 * most tokens; abstract page: keys and values are linear combinations of
 * static dictionary vectors). For batch b and query head h (KV head
 * g = h / (Hq/Hkv)):
 *   u       = scale * Dk q_h                                   [n_atoms]
 *   s_low_t = sum_{j<klow}  kappa_tj u[i_tj]                   all t < T
 *   S       = the m = ceil(T*top_num/top_den) tokens with largest s_low,
 *             ties to the lower token index
 *   s_high_t= sum_{j<khigh} kappa_tj u[i_tj]                   t in S
 *   p       = softmax_S(s_high);  w[a] = sum_{t in S} p_t sum_{j<K}
 *             kappa^v_tj [i^v_tj == a];  out_h = Dv^T w
 * Unselected tokens do not enter the softmax.
 * ---------------------------------------------------------------------- */
typedef struct sdkv_attn_args {
  const void* q;        /* [B, Hq, d] queries, q_dtype SDKV_BF16 or
                           SDKV_F32 (fp32 values are split exactly into
                           three bf16 parts on the matrix cores)          */
  int32_t q_dtype;
  const void* dk;       /* [n_atoms, d] key dictionary, dict_dtype        */
  const void* dv;       /* [n_atoms, d] value dictionary, dict_dtype      */
  int32_t dict_dtype;
  int32_t n_atoms;      /* 1 .. 32768                                     */
  int32_t B, Hq, Hkv;   /* >= 1, Hq % Hkv == 0                            */
  int32_t d;            /* 64 or 128                                      */
  int64_t T;            /* cached tokens, >= 1                            */
  const uint32_t* key_low;   /* [B, Hkv, T, klow] first klow key words, or
                                NULL to read them from key_codes          */
  const uint32_t* key_codes; /* [B, Hkv, T] records of K key code words    */
  const uint32_t* val_codes; /* [B, Hkv, T] records of K value code words  */
  int64_t code_stride;  /* words from one token's record to the next, in
                           both key_codes and val_codes: 0 means K (dense
                           [B, Hkv, T, K] arrays); 2K with val_codes =
                           key_codes + K stores each token's key and value
                           records side by side ([B, Hkv, T, 2, K]), so
                           that both come in one 128-byte line at K = 16.
                           Must be 0 or in [K, 65536].                    */
  int32_t K;            /* 1 .. 32                                        */
  int32_t klow, khigh;  /* 1 <= klow <= khigh <= K                        */
  int64_t top_num, top_den; /* selected fraction, 0 < top_num <= top_den  */
  float scale;          /* softmax scale, finite                          */
  float* out;           /* OUT [B, Hq, d] fp32; required                  */
  /* Optional per-stage outputs (NULL to skip):                           */
  float* u;             /* OUT [B, Hq, n_atoms] scale * Dk q              */
  float* s_low;         /* OUT [B, Hq, T]                                 */
  int32_t* sel;         /* OUT [B, Hq, m] selected tokens, ascending      */
  float* s_high;        /* OUT [B, Hq, m] aligned with sel                */
  float* w;             /* OUT [B, Hq, n_atoms] normalised value weights  */
  /* Optional stage timing: NULL, or SDKV_DECODE_STAGES + 1 hipEvent_t
     handles (created by the caller); event i is recorded on `stream` before
     stage i and the last one after the final stage. Stages: 0 U table,
     1 score/select/rescore/softmax/value weights, 2 W.Dv contraction,
     3 output reduction. A failed event record returns SDKV_ERR_DEVICE.   */
  void* const* stage_events;
  /* Softmax over the selected tokens (review page, Summary and Strengths:
     the integer-only execution; Table 1 and Section 3.1.3 on token-wise
     INT16 requantization at the Softmax input):
       SDKV_SOFTMAX_FLOAT (0): fp32 exp, as above.
       SDKV_SOFTMAX_INT   (1): integer-only. Per row (b, h), with A the
         largest |s_high| over S, k = clamp(15 - E, 1, 30) where A = f 2^E,
         f in [0.5, 1) (k = 30 when A = 0):
           q_t  = clamp(rint(s_high_t 2^k), -32767, 32767) - max_S q
           exp: X = -q_t 2^(30-k); z = floor(X / LN2); qp = -((X - z LN2)
                >> (30-k)); t = (qp + (B >> (30-k))) >> g, g = max(0, k-14);
                e_t = (t^2 + (CA >> (30 - 2(k-g)))) >> z, 0 once z >= 31;
                LN2 = 744261117, B = 1452772687, CA = 1030312935 (ln 2,
                1.353 and 0.344/0.3585 with 30 fractional bits, floor:
                I-BERT's fit exp(p) ~ 0.3585 (p + 1.353)^2 + 0.344)
           guard: h = max(0, bitlen(m) + bitlen(e_max) - 30), e_max the
                value at q = 0; e'_t = (e_t + 2^(h-1)) >> h (h > 0)
           p_t = (e'_t floor(2^62 / sum_S e')) >> 32   (30 fractional bits)
         and w[a] = sum_t (p_t / 2^30) kappa^v ... as above.
       Other values: SDKV_ERR_SHAPE.                                      */
  int32_t softmax_mode;
  int32_t* p_int;       /* OUT [B, Hq, m] integer p_t aligned with sel
                           (SDKV_SOFTMAX_INT only), or NULL               */
  /* Selection granularity under grouped-query attention (review page,
     Summary: the selection is query-aware; the pages are silent on GQA):
       SDKV_SELECT_HEAD (0): every query head ranks the tokens by its own
         s_low, as above.
       SDKV_SELECT_KV   (1): the G = Hq/Hkv query heads of a KV head share
         one selection, ranked by their summed low score
         sum_{j<klow} kappa_tj U_g[i_tj], U_g = sum_{h in g} u_h (fp32, h
         ascending); s_high, the softmax and w stay per head. The s_low
         debug output then holds that shared score for every head.
       Other values: SDKV_ERR_SHAPE.                                      */
  int32_t select_mode;
  /* Which tokens enter the softmax (review page, Summary: every token is
     scored with Klow atoms and the best tenth refined with Khigh; the pages
     do not say whether the rest then drop out):
       SDKV_READING_A (0): only S, as above.
       SDKV_READING_B (1): every token; t in S with s_high_t and its K value
         pairs, t not in S with its own head's s_low_t and its first klow
         value pairs:  p = softmax over all T,
           w[a] = sum_{t in S} p_t sum_{j<K} kappa^v_tj [i^v_tj == a]
                + sum_{t not in S} p_t sum_{j<klow} kappa^v_tj [i^v_tj == a].
         Requires SDKV_SOFTMAX_FLOAT (else SDKV_ERR_UNSUPPORTED).
       Other values: SDKV_ERR_SHAPE.                                      */
  int32_t reading;
  const uint32_t* val_low; /* [B, Hkv, T, klow] first klow value words, or
                              NULL to read them from val_codes (reading B) */
} sdkv_attn_args;
#define SDKV_DECODE_STAGES 4
#define SDKV_SOFTMAX_FLOAT 0
#define SDKV_SOFTMAX_INT 1
#define SDKV_SELECT_HEAD 0
#define SDKV_SELECT_KV 1
#define SDKV_READING_A 0
#define SDKV_READING_B 1

/* m = ceil(T * top_num / top_den), clamped to [1, T]; 0 on bad input. */
SDKV_API int64_t sdkv_selected_count(int64_t T, int64_t top_num, int64_t top_den);

SDKV_API sdkv_status sdkv_decode_attn_workspace(const sdkv_attn_args* args, size_t* bytes);
SDKV_API sdkv_status sdkv_decode_attn(const sdkv_attn_args* args, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Top-k select: the "top 10%" step of the decode path on its own (review
 * page, Summary). For each of `rows` rows of `n` fp32 scores (row stride
 * `ld` elements, ld >= n), writes the indices of the k largest scores,
 * ties to the lower index, in ascending index order: idx_out [rows, k].
 * thr_out (nullable) [rows] receives the k-th largest score.
 * Limits: 1 <= k <= n <= 2^23.
 * ---------------------------------------------------------------------- */
SDKV_API sdkv_status sdkv_select_topk_workspace(int64_t rows, int64_t n, int64_t k,
                                       size_t* bytes);
SDKV_API sdkv_status sdkv_select_topk(const float* scores, int64_t rows, int64_t n,
                             int64_t ld, int64_t k, int32_t* idx_out,
                             float* thr_out, void* ws, size_t ws_bytes,
                             void* stream);

SDKV_API const char* sdkv_status_str(sdkv_status s);
SDKV_API int32_t sdkv_abi_version(void);

/* Test hook, for tests of the wait-failure path only: every later call's
 * cross-workgroup waits give up after `polls` polls (0 restores the normal
 * bound) and wait for `extra` more arrivals than exist (0 in normal use).
 * With extra > 0 every wait gives up, the kernels select nothing from
 * exchanged data and still exit normally, and the status word reads 1.
 * Process-wide; not for concurrent use with other calls. */
SDKV_API void sdkv_test_set_wait(uint32_t polls, uint32_t extra);

#ifdef __cplusplus
}
#endif
#endif /* SDKV_H */
