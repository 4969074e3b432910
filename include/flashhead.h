/*
 * flashhead.h -- C ABI of the FlashHead output head for AMD Instinct MI355X (gfx950).
 *
 * FlashHead ("FlashHead: Efficient Drop-In Replacement for the Classification Head in
 * Language Model Inference", Section 3) replaces the dense LM head z = E h (E: [V][d])
 * by retrieval over balanced vocabulary clusters:
 *   1. offline, the V token embeddings are split into c clusters of exactly b = V / c
 *      tokens by balanced spherical k-means (Section 3.1); C[c][d] holds the centroids
 *      and C2T[c][b] the token ids of each cluster;
 *   2. online, the centroid logits C h are computed, p clusters are kept -- the top p
 *      (greedy) or p drawn without replacement from softmax(C h / tau) (sampling) -- the
 *      tokens of those clusters are gathered, their logits computed, and the argmax or a
 *      sample from their softmax is returned (Section 3.2).
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are device memory of the current HIP device; "host"
 *     pointers are host memory.  The caller owns every buffer; the library never keeps a
 *     pointer after a call returns and never allocates on the forward path.
 *   - Arrays are dense and row-major with the shapes given; element types follow the
 *     fh_dtype fields of fh_desc.  bf16 values are passed as their 16-bit patterns.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous: results are valid once the stream has been synchronised.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - All argument and shape checks run on the host before anything is enqueued.  A check
 *     that fails returns its status, enqueues nothing and sets the message returned by
 *     flashhead_last_error() (thread-local).  A HIP launch error returns FH_ERR_HIP.
 *   - Device data are not validated on the forward path: ids in C2T must form a
 *     permutation of [0, V) (flashhead_pack checks this), and NaN inputs give an
 *     unspecified (but in-bounds) result.
 *   - Ties: a larger key wins; equal keys go to the smaller cluster id (probe selection)
 *     or to the smaller vocabulary id (token choice), so p = c reproduces the dense head.
 *
 * Random numbers (sampling mode).  Philox4x32-10 (Salmon et al., SC'11) with
 *   key = (seed mod 2^32, seed >> 32), counter = (n >> 2, row, step mod 2^32,
 *   ((step >> 32) << 2) | stream), word n & 3, u = (2 (word >> 9) + 1) 2^-24,
 *   Gumbel noise G = -ln(-ln u).
 * Stream 0 draws the cluster keys (n = cluster id), stream 1 the token keys (n =
 * vocabulary id); row is the row of h within the call.
 */
#ifndef FLASHHEAD_H_
#define FLASHHEAD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLASHHEAD_ABI_VERSION 1

typedef enum fh_status {
    FH_OK = 0,
    FH_ERR_ARG = 1,          /* null pointer, bad enum value, p out of range, tau <= 0 */
    FH_ERR_SHAPE = 2,        /* V not a multiple of c, d not a multiple of 8 (128 for int4) */
    FH_ERR_DTYPE = 3,        /* dtype combination not accepted by this entry point */
    FH_ERR_UNSUPPORTED = 4,  /* shape beyond this build's limits (see flashhead_forward) */
    FH_ERR_WORKSPACE = 5,    /* workspace missing or smaller than the *_workspace_bytes size */
    FH_ERR_HIP = 6           /* a HIP runtime call failed; the message names it */
} fh_status;

typedef enum fh_dtype {
    FH_F32 = 0,              /* IEEE float32 */
    FH_BF16 = 1,             /* bfloat16 bit patterns (uint16) */
    FH_INT4_G128 = 2         /* token embeddings only: int4 with a bf16 scale per 128 elements */
} fh_dtype;

typedef enum fh_mode {
    FH_GREEDY = 0,           /* top-p clusters by centroid logit, then argmax of the gathered logits */
    FH_SAMPLE = 1            /* Gumbel-top-p clusters, then a Gumbel-max token sample, both at tau */
} fh_mode;

/* Shapes and element types of one head. */
typedef struct fh_desc {
    int64_t B;               /* rows of h per call, >= 1 */
    int64_t d;               /* hidden size */
    int64_t V;               /* vocabulary size */
    int64_t c;               /* clusters; b = V / c tokens per cluster */
    int32_t h_dtype;         /* FH_F32 | FH_BF16 */
    int32_t c_dtype;         /* FH_F32 | FH_BF16 | FH_INT4_G128 (centroids) */
    int32_t e_dtype;         /* FH_F32 | FH_BF16 | FH_INT4_G128 (token embeddings / tiles) */
    int32_t reserved;        /* must be 0 */
} fh_desc;

/* Outputs of a forward call; every pointer is device memory.  Only `token` is required. */
typedef struct fh_outputs {
    int32_t* token;          /* [B] chosen vocabulary id per row */
    int32_t* probe_ids;      /* [B][p] kept clusters, ascending cluster id; may be NULL */
    float*   probe_logits;   /* [B][p][b] logit of token j of the q-th kept cluster; may be NULL */
    int32_t* probe_tokens;   /* [B][p][b] vocabulary id of that token (C2T row); may be NULL */
} fh_outputs;

/* Library version string, e.g. "flashhead 0.1.0 gfx950". */
const char* flashhead_version(void);

/* Message describing the last non-FH_OK status returned on the calling thread. */
const char* flashhead_last_error(void);

/*
 * Workspace size (bytes, device memory) that flashhead_forward and the stage entry points
 * need for this desc and p.  Writes it to *bytes (host).  The workspace carries
 * the centroid keys, probe lists and per-row maxima between the stages of one call; it
 * needs no initialisation.
 */
fh_status flashhead_workspace_bytes(const fh_desc* desc, int64_t p, size_t* bytes);

/*
 * Offline packing into cluster-major tiles (the paper's dense C2T of Section 3.2,
 * "Complexity": equal cluster sizes make the tokens of cluster k a fixed-size block).
 *   E              device, [V][d] token-major embeddings of dtype src_dtype (F32 | BF16)
 *   cluster_tokens device, int32 [c][b]: C2T, a permutation of [0, V)
 *   E_tiles        device out: row (k, j) = E[C2T[k][j]] at offset (k b + j) * row size,
 *                  in desc->e_dtype: F32 / BF16 rows of d values (f32 -> bf16 rounds to
 *                  nearest even), or INT4_G128 rows of d/2 bytes (element 2i in the low
 *                  nibble of byte i, two's complement, q = clamp(rne(x / s), -7, 7))
 *   E_scales       device out, INT4_G128 only: bf16 [c][b][d/128], s = bf16(amax / 7) of each
 *                  group of 128 elements (s = 0 and q = 0 for an all-zero group); else NULL
 * The low-bit format is this library's reading of the paper's selective quantization
 * (Section 3.2, "Quantization note"; Table 5).
 * Unequal clusters (the ablation of Sections 3.1 and 4.5, Table 6): C2T keeps its dense
 * [c][b] shape with b = the largest cluster and -1 in the empty slots of smaller clusters
 * (desc->V = c b slots); an empty slot gets a zero row.  Checks that the entries other than -1
 * are the tokens 0 .. n-1 once each (n = the slots that are not empty; with equal clusters a
 * permutation of [0, V)): FH_ERR_ARG if not.  This call allocates a small device buffer and
 * synchronises `stream`.
 */
fh_status flashhead_pack(const fh_desc* desc, int32_t src_dtype, const void* E,
                         const int32_t* cluster_tokens, void* E_tiles, void* E_scales,
                         void* stream);

/*
 * Offline balanced spherical k-means (Section 3.1, "Clustering the Embedding Matrix"): c
 * clusters of exactly b = V / c tokens each.  Rows are normalised; the centres start from
 * k-means++ in the spherical metric (weights 2 - 2 cos; draw m uses Philox4x32-10 keyed by
 * `seed`, stream 2, row 0, step m, element 0, by inverse CDF over the weight prefix sums in
 * ascending token id); each of `iters` rounds assigns every token its most similar centre,
 * lets an over-full cluster keep its b most similar members (ties: smaller token id) and
 * places the evicted tokens, in ascending id, on the most similar cluster with room (ties:
 * smaller cluster id), then sets c_k = normalise(sum of the members' unit rows).  The page
 * fixes neither the initialisation, the iteration count nor these orders; they are this
 * library's readings.  All arithmetic is fp64 with fixed reduction orders and stable
 * sorts, so the result does not depend on scheduling.
 *   desc           V, d, c (b = V / c <= 256, c <= 32768); desc->c_dtype: stored centroids
 *                  (F32 | BF16)
 *   src_dtype      dtype of E (F32 | BF16)
 *   E              device, [V][d] token-major embeddings
 *   iters          >= 1 rounds
 *   unit           0: stored centroid = mean of the members' raw rows (as flashhead_centroids);
 *                  1: the unit centroid c_k of the last round
 *   centroids      device out, [c][d] in desc->c_dtype (rounded once, to nearest even)
 *   cluster_tokens device out, int32 [c][b]: C2T, members in ascending token id
 *   workspace      device, >= flashhead_build_clusters_workspace_bytes (about 8 V d bytes)
 * Offline: launches thousands of kernels (two per k-means++ draw) and synchronises
 * `stream` once per round.
 */
fh_status flashhead_build_clusters_workspace_bytes(const fh_desc* desc, int32_t src_dtype, size_t* bytes);
fh_status flashhead_build_clusters(const fh_desc* desc, int32_t src_dtype, const void* E, int32_t iters,
                                   uint64_t seed, int32_t unit, void* centroids, int32_t* cluster_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the centroid buffer for desc->c_dtype: c d 4 (F32), c d 2 (BF16), or for
 * INT4_G128 (the paper's stage-1 quantisation, Section 4.5, Table 5) the nibbles
 * [c][d/2] (element 2i in the low nibble of byte i) followed, at byte offset
 * round_up(c d / 2, 256), by the bf16 group scales [c][d/128].  Writes it to *bytes.
 */
fh_status flashhead_centroids_bytes(const fh_desc* desc, size_t* bytes);

/*
 * Offline centroids of a given clustering (Section 3.1, "Centroid matrix").
 *   E              device, [V][d] token-major embeddings of dtype src_dtype (F32 | BF16)
 *   cluster_tokens device, int32 [c][b]: C2T (entries -1: empty slots of a padded C2T, see
 *                  flashhead_pack, which are not members; a cluster without members gets 0)
 *   unit           0: C[k] = mean of the member rows of cluster k;
 *                  1: C[k] = normalise(sum of the normalised rows), the unit centroid the
 *                     paper stores (a zero row or sum contributes / gives 0)
 *   centroids      device out, [c][d] in desc->c_dtype (layout: flashhead_centroids_bytes)
 * Sums run in fp64 and are rounded once to the output dtype (bf16: nearest even).  The
 * forward pass accepts either form.  INT4_G128: the bf16 centroids, quantised per group of
 * 128 exactly like int4 token rows (s = bf16(amax / 7), q = clamp(rne(x / s), -7, 7)); this
 * case allocates a temporary buffer and synchronises `stream`.  Otherwise asynchronous.
 */
fh_status flashhead_centroids(const fh_desc* desc, int32_t src_dtype, const void* E,
                              const int32_t* cluster_tokens, int32_t unit, void* centroids,
                              void* stream);

/*
 * Stage 1 (Section 3.2): centroid logits s[r][k] = sum_j h[r][j] C[k][j], fp32 accumulation,
 * turned into probe keys -- s (greedy) or s / tau + G(U(seed, r, step, 0, k)) (sampling) --
 * stored in the workspace and, if keys_out (device, float [B][c]) is non-NULL, there too.
 *   h         device [B][d], desc->h_dtype
 *   centroids device [c][d], desc->c_dtype (INT4_G128 layout: flashhead_centroids_bytes)
 */
fh_status flashhead_centroid_scores(const fh_desc* desc, const void* h, const void* centroids,
                                    int32_t mode, float temperature, uint64_t seed, uint64_t step,
                                    void* workspace, size_t workspace_bytes, float* keys_out,
                                    void* stream);

/*
 * Probe selection (Section 3.2): for every row keep the p clusters with the largest stage-1
 * keys (ties to the smaller cluster id).  With sampling keys this is Gumbel-top-p, i.e. p
 * clusters drawn without replacement from softmax(s / tau).  Reads the keys the last
 * flashhead_centroid_scores call left in `workspace`; writes the kept ids, ascending, to
 * the workspace and, if probe_ids_out (device, int32 [B][p]) is non-NULL, there too.  At
 * B > 1 the selection also records, per cluster, the rows that kept it (cleared first by
 * this call, so selections may follow each other on one workspace with any p).
 */
fh_status flashhead_select_probes(const fh_desc* desc, int64_t p, void* workspace,
                                  size_t workspace_bytes, int32_t* probe_ids_out, void* stream);

/*
 * Stage 2 (Section 3.2): for every kept cluster k of every row r, the logits
 * z = E_tiles[k][j] . h[r] (j < b, fp32 accumulation; int4 rows are dequantised to q s)
 * and the token choice: argmax z (greedy) or argmax z / tau + G(U(seed, r, step, 1, t)),
 * t = C2T[k][j] (sampling, a Gumbel-max draw from softmax(z / tau) over the gathered
 * tokens).  Reads the probe lists the last flashhead_select_probes call left in
 * `workspace`.  Writes out->token and the optional outputs.
 *   cluster_tokens device int32 [c][b]; E_tiles / E_scales as written by flashhead_pack.
 */
fh_status flashhead_probe_logits(const fh_desc* desc, int64_t p, const void* h,
                                 const int32_t* cluster_tokens, const void* E_tiles,
                                 const void* E_scales, int32_t mode, float temperature,
                                 uint64_t seed, uint64_t step, void* workspace,
                                 size_t workspace_bytes, const fh_outputs* out, void* stream);

/*
 * Probe selection and stage 2 in one call: the same results as flashhead_select_probes
 * followed by flashhead_probe_logits (out->probe_ids receives the kept ids, ascending, if
 * non-NULL).  Reads the keys the last flashhead_centroid_scores call left in `workspace`, so
 * flashhead_centroid_scores + flashhead_select_and_probe is flashhead_forward.  At B = 1 the
 * selection and the probed logits run in one kernel: every workgroup selects the same kept
 * set and scores its share of it, from per-group candidate lists that stage 1 also leaves in
 * the workspace (each group of consecutive clusters lists its largest keys; the selection over
 * the lists is exact and falls back to all c keys when a list may have been cut short).
 * Arguments as for flashhead_probe_logits.
 */
fh_status flashhead_select_and_probe(const fh_desc* desc, int64_t p, const void* h,
                                     const int32_t* cluster_tokens, const void* E_tiles,
                                     const void* E_scales, int32_t mode, float temperature,
                                     uint64_t seed, uint64_t step, void* workspace,
                                     size_t workspace_bytes, const fh_outputs* out, void* stream);

/*
 * The whole head: stage 1, probe selection and stage 2 as above, enqueued back to back
 * (flashhead_centroid_scores, then flashhead_select_and_probe).
 *   h              device [B][d]
 *   centroids      device [c][d] in desc->c_dtype (INT4_G128 layout: flashhead_centroids_bytes)
 *   cluster_tokens device int32 [c][b]
 *   E_tiles        device, cluster-major tiles (flashhead_pack)
 *   E_scales       device, INT4_G128 scales, else NULL
 *   p              1 <= p <= c
 *   mode           FH_GREEDY | FH_SAMPLE; temperature > 0 (sampling only), applied to both
 *                  stages; seed / step key the Philox draws
 *   workspace      device, >= flashhead_workspace_bytes(desc, p)
 *   out            host struct of device pointers
 * An empty slot of a padded C2T (entry -1, see flashhead_pack) gathers nothing: it is never the
 * token, and out->probe_tokens / probe_logits report it as -1 / -inf.
 * Limits of this build: d % 8 == 0, d <= 4096 (bf16 rows), <= 2048 (f32 rows), d % 128 == 0
 * and d <= 8192 (int4 rows), each bound applying to both the centroids' and the tiles' format
 * (so d > 4096 needs int4 centroids and int4 tiles); c <= 32768; 1 <= b <= 256; V < 2^31;
 * B <= 65535.  Beyond them the call returns FH_ERR_UNSUPPORTED before any launch.
 */
fh_status flashhead_forward(const fh_desc* desc, const void* h, const void* centroids,
                            const int32_t* cluster_tokens, const void* E_tiles,
                            const void* E_scales, int64_t p, int32_t mode, float temperature,
                            uint64_t seed, uint64_t step, void* workspace, size_t workspace_bytes,
                            const fh_outputs* out, void* stream);

/*
 * flashhead_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a static scratch array inside the library, one per device, of 4 MiB (4194304
 * bytes), held until the process ends.  Arguments,
 * results and errors as for flashhead_forward; a head whose workspace
 * (flashhead_workspace_bytes) exceeds the scratch returns FH_ERR_UNSUPPORTED.  Every call on a
 * device shares that device's scratch: calls that overlap in time on one device (other streams,
 * other threads) race and give undefined results; calls ordered on one stream are safe.  The
 * first call on a device looks up the scratch's device address (no allocation); nothing here
 * calls hipMalloc or hipFree.
 */
fh_status flashhead_forward_noalloc(const fh_desc* desc, const void* h, const void* centroids,
                                    const int32_t* cluster_tokens, const void* E_tiles,
                                    const void* E_scales, int64_t p, int32_t mode, float temperature,
                                    uint64_t seed, uint64_t step, const fh_outputs* out, void* stream);

/* Workspace size (bytes, device memory) for flashhead_mc_marginal. */
fh_status flashhead_mc_marginal_workspace_bytes(const fh_desc* desc, size_t* bytes);

/*
 * Monte-Carlo estimate of the two-stage sampler's distribution over the whole vocabulary
 * (Appendix D.1, "Monte-Carlo Simulation"): for probe sets S_0 .. S_{N-1}, N = n_sets, drawn
 * as the sampler's stage 1 draws them -- S_i is the Gumbel-top-p set of the keys
 * s / tau + G(U(seed, r, step = i, 0, k)), i.e. flashhead_forward's probe set at step i --
 *   out[r][v] = (1 / N) sum_i p(v | h_r, S_i),
 * p(v | h, S) the softmax of z / tau over the tokens of the clusters in S (0 for the
 * others).  With clip = 1 every zero entry of a row (a token no S_i reached) is replaced
 * by the row's smallest non-zero entry, as the appendix does before taking logarithms.
 *   h, centroids, cluster_tokens, E_tiles, E_scales, p   as for flashhead_forward
 *   temperature    > 0, used by both stages
 *   n_sets         1 <= n_sets < 2^31
 *   clip           0 | 1
 *   workspace      device, >= flashhead_mc_marginal_workspace_bytes(desc)
 *   out            device double [B][V], indexed by vocabulary id
 * It needs equal clusters (a C2T without empty slots); the empty slots of a padded C2T are
 * never written in `out`, but the estimate does not exclude them.
 * The logits s and z are computed with fp32 accumulation (s as flashhead_centroid_scores;
 * z over the whole tile array, as flashhead_dense_forward for bf16 / fp32 tiles and as
 * flashhead_probe_logits for int4 tiles); the softmax statistics and the average are fp64,
 * accumulated with atomic adds whose order varies between runs (the last bits of `out` may
 * too).
 */
fh_status flashhead_mc_marginal(const fh_desc* desc, const void* h, const void* centroids,
                                const int32_t* cluster_tokens, const void* E_tiles, const void* E_scales,
                                int64_t p, float temperature, uint64_t seed, int64_t n_sets, int32_t clip,
                                void* workspace, size_t workspace_bytes, double* out, void* stream);

/* Workspace size (bytes) for flashhead_dense_forward. */
fh_status flashhead_dense_workspace_bytes(const fh_desc* desc, size_t* bytes);

/*
 * The dense head the paper starts from (Section 3): z = E h over all V tokens, then argmax
 * (greedy) or argmax z / tau + G(U(seed, r, step, 1, t)) (sampling), ties to the smaller id.
 * The same token keys as flashhead_forward's stage 2 (the same noise on logits that agree up
 * to fp32 rounding), so p = c gives the same token unless the top two keys are that close.
 *   E       device [V][d] token-major, desc->e_dtype F32 | BF16 | INT4_G128; INT4_G128 is one
 *           buffer: the nibbles [V][d/2] (the tile format of flashhead_pack), then from byte
 *           round_up(V d / 2, 256) the bf16 group scales [V][d/128] -- the layout
 *           flashhead_centroids writes, so a c = V, b = 1 call with C2T[t][0] = t quantises E
 *           (the dense head of the paper's quantisation comparison, Section 4.5, Table 5)
 *   token   device int32 [B] out
 *   logits  device float [B][V] out, may be NULL
 */
fh_status flashhead_dense_forward(const fh_desc* desc, const void* h, const void* E,
                                  int32_t mode, float temperature, uint64_t seed, uint64_t step,
                                  void* workspace, size_t workspace_bytes, int32_t* token,
                                  float* logits, void* stream);

/*
 * The sampler's random numbers exactly as the kernels draw them (the Philox4x32-10 counter
 * layout above; Section 3.2 samples clusters and tokens but fixes no generator), for checking
 * the generator against another implementation:
 *   words_out[i]  = the Philox word of element n = n0 + i of (seed, row, step, rng_stream)
 *   gumbel_out[i] = G(u) = -ln(-ln u) in fp32 (logf), u = (2 (word >> 9) + 1) 2^-24
 * Either output may be NULL (not both); both are device arrays of `count` elements.
 * rng_stream 0 .. 3; count >= 0 with n0 + count <= 2^32, else FH_ERR_ARG.
 */
fh_status flashhead_philox_words(uint64_t seed, uint32_t row, uint64_t step, uint32_t rng_stream,
                                 uint32_t n0, int64_t count, uint32_t* words_out, float* gumbel_out,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHHEAD_H_ */
