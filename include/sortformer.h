/*
 * sortformer.h — C ABI of the MI355X (gfx950) Streaming Sortformer /
 * Nemotron-3-style speaker-diarization forward.
 *
 * The library computes, on one GPU, the frame-classification forward the
 * pages describe: 128-bin log-mel frontend, 8x ConvSubsampling (pre_encode),
 * 17 FastConformer layers, encoder_proj, 18 Transformer layers and a sigmoid
 * speaker head ("Streaming Sortformer Diarizer" model card, Pipeline), run
 * over the [speaker_cache | FIFO | chunk] window with FIFO pops and log-odds
 * speaker-cache compression (same card, Streaming Architecture). The
 * Nemotron-3-style variant (8x stacked mel, 31 RoPE transformer layers,
 * 8 speakers, ConvTranspose 10 ms head) follows the model-card summary in
 * the ExecuTorch issue "Enable Nemotron-3-Diarization on MLX, CUDA, XNNPACK,
 * and Vulkan".
 *
 * Conventions for every call:
 *  - Pointers prefixed d_ are device (HIP) pointers; all others are host.
 *  - The caller allocates every device buffer (weights, workspace, state)
 *    with the sizes the *_bytes queries return; the library never keeps a
 *    reference to caller host memory after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Compute calls only enqueue work on that stream and return without
 *    waiting for it, unless documented otherwise.
 *  - Every call returns an sf_status; on error nothing is enqueued and
 *    caller outputs are left untouched. HIP errors are mapped to SF_EHIP,
 *    never thrown. Calls on one model/stream object are not thread-safe.
 *  - Tensors are row-major, batch-major: (B, rows, cols), fp32 unless stated.
 */
#ifndef SORTFORMER_H
#define SORTFORMER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sf_status;
#define SF_OK 0
#define SF_EINVAL (-1)        /* bad argument (null pointer, unknown enum)      */
#define SF_ESHAPE (-2)        /* size outside the supported range               */
#define SF_ENOMEM (-3)        /* caller buffer smaller than the size query      */
#define SF_EHIP (-4)          /* a HIP runtime call failed                      */
#define SF_ESTATE (-5)        /* call not allowed in the stream's current state */
#define SF_EUNSUPPORTED (-6)  /* combination not implemented                    */

#define SF_ARCH_SORTFORMER 0  /* 4 speakers, conformer + transformer, 80 ms out */
#define SF_ARCH_NEMOTRON 1    /* 8 speakers, RoPE transformer, 10 ms out        */
#define SF_DTYPE_F32 0        /* every GEMM operand fp32                         */
#define SF_DTYPE_BF16 1       /* GEMM/attention operands bf16, fp32 accumulate   */
#define SF_INIT_SPEC 0        /* weights N(0,0.02^2), biases 0, norms gamma 1    */
#define SF_INIT_FULL_RANDOM 1 /* also biases/norm params/BN stats random        */

/* Longest encoder window (frames of 80 ms) any call accepts; the relative
 * position and rotary tables are sized for it. The pages' own exported
 * encoder accepts at most 1000 frames (model card, Exported Methods). */
#define SF_MAX_WINDOW 1024

typedef struct sf_model_config {
  int32_t arch;      /* SF_ARCH_*                                 */
  int32_t dtype;     /* SF_DTYPE_*                                */
  int32_t init_mode; /* SF_INIT_*                                 */
  int32_t n_spk;     /* 4 for SORTFORMER, 8 for NEMOTRON (checked) */
} sf_model_config;

/* Streaming window configuration, all in 80 ms encoder frames (model card,
 * Streaming Configurations; latency = (chunk_len + right_context) x 80 ms). */
typedef struct sf_stream_config {
  int32_t chunk_len;     /* frames scored per step                           */
  int32_t right_context; /* look-ahead frames attended but not scored        */
  int32_t fifo_len;      /* FIFO capacity before frames pop into the cache   */
  int32_t update_period; /* minimum frames popped per overflow               */
  int32_t spkcache_len;  /* speaker-cache size after compression (188)       */
  int32_t n_sil_per_spk; /* silence placeholders guaranteed per speaker (3)  */
} sf_stream_config;

typedef struct sf_model sf_model;   /* opaque, host-side */
typedef struct sf_stream sf_stream; /* opaque, host-side */

/* Human-readable text for a status code (static storage). */
const char* sortformer_status_string(sf_status status);

/* Named presets: "very_high" 340/40/40/300/188, "high" 124/1/124/124/188,
 * "low" 6/7/188/144/188, "ultra_low" 3/1/188/144/188 (model card, Streaming
 * Configurations), "very_low" 6/2/188/144/188 (the 0.64 s streaming mode of
 * the Transformers docs "Nemotron 3 Diarization", whose chunk / look-ahead
 * split is not given: read as Low's chunk with a 2-frame look-ahead) and
 * "nemotron_offline" 380/0/188/192/188 (30.4 s chunks, same docs, Overview).
 * SF_EINVAL if the name is unknown. */
sf_status sortformer_stream_preset(const char* name, sf_stream_config* out);

/* ------------------------------------------------------------------ model */

/* Device bytes the weights (plus derived tables) need; 0 if cfg is invalid.
 * The tensors are those of the "Streaming Sortformer Diarizer" model card's
 * Pipeline and Model Parameters (117M parameters, about 470 MB in fp32), or of
 * the Nemotron-3-Diarization summary in the ExecuTorch issue (about 100M). */
size_t sortformer_weight_bytes(const sf_model_config* cfg);

/* The model with seeded random weights: the pages run a trained checkpoint
 * ("Streaming Sortformer Diarizer" model card, Pipeline; Transformers docs,
 * Overview), which does not exist here, so every weight is drawn instead.
 * Generates them on the host (SplitMix64 counters + Box-Muller, one stream
 * per tensor), uploads them into d_weights (caller memory of >=
 * sortformer_weight_bytes bytes, 256-byte aligned), derives the device tables
 * (relative-position projections, folded BatchNorm, DFT/mel tables) and
 * returns a host handle in *out. Blocks until the uploads are done.
 * d_weights must stay allocated until sortformer_free. Errors: SF_EINVAL
 * (null pointer, invalid cfg, misaligned d_weights), SF_ENOMEM
 * (weight_bytes too small), SF_EHIP. */
sf_status sortformer_init(const sf_model_config* cfg, uint64_t seed, void* d_weights,
                          size_t weight_bytes, void* stream, sf_model** out);
/* Releases the host handle (the caller frees d_weights afterwards). NULL is
 * ignored. */
void sortformer_free(sf_model* model);
/* The configuration the model was created with. SF_EINVAL on null pointers. */
sf_status sortformer_get_config(const sf_model* model, sf_model_config* out);

/* Model options.
 * SF_OPT_OUTPUT_STRIDE (NEMOTRON): output frames of value x 10 ms, value in
 *   {1, 2, 4, 8} (default 1, the head's 10 ms frames). The Transformers docs
 *   "Nemotron 3 Diarization" (Overview) give the output frame resolution as
 *   configurable in 10 ms steps with one checkpoint, and the model-card
 *   summary in the ExecuTorch issue 10 ms as the default; the pages do not
 *   say how a coarser frame is formed. Here output frame k is the mean of
 *   the head's 10 ms probabilities value*k .. value*k + value - 1, and value
 *   divides 8 so every 80 ms encoder frame holds a whole number of output
 *   frames. Read by every later offline call and stream step of the model
 *   (sortformer_stream_max_emit reflects it). SORTFORMER accepts only 1
 *   (SF_EUNSUPPORTED otherwise); other values give SF_EINVAL. */
#define SF_OPT_OUTPUT_STRIDE 1
sf_status sortformer_set_option(sf_model* model, int32_t option, int32_t value);
/* Current value of a model option (-1 for an unknown option or null model). */
int32_t sortformer_get_option(const sf_model* model, int32_t option);

/* Model metadata: the constants the "Streaming Sortformer Diarizer" model
 * card exports beside its methods (Exported Methods, Metadata:
 * sample_rate, window_stride, subsampling_factor, fc_d_model, tf_d_model,
 * max_num_of_spks, spkcache_len) and the frontend and layer sizes of the
 * same card's Pipeline and Model Parameters. For NEMOTRON the encoder is the
 * 31-layer rotary Transformer of width 512 (no FastConformer: fc_d_model 0)
 * and the output runs at 10 ms. */
typedef struct sf_model_metadata {
  double window_stride;         /* seconds between mel frames: 0.01              */
  double output_frame_s;        /* seconds per output frame: 0.08 or 0.01         */
  int32_t sample_rate;          /* 16000                                          */
  int32_t subsampling_factor;   /* mel frames per encoder frame: 8                */
  int32_t fc_d_model;           /* FastConformer width: 512 (SORTFORMER), 0       */
  int32_t tf_d_model;           /* Transformer width: 192 (SORTFORMER), 512       */
  int32_t max_num_of_spks;      /* 4 (SORTFORMER), 8 (NEMOTRON)                   */
  int32_t spkcache_len;         /* speaker-cache frames of every preset: 188      */
  int32_t n_mels, n_fft, win_length, hop_length; /* 128, 512, 400, 160          */
  int32_t n_conformer_layers;   /* 17 (SORTFORMER), 0                             */
  int32_t n_transformer_layers; /* 18 (SORTFORMER), 31 (NEMOTRON)                 */
  int32_t n_heads;              /* 8                                              */
  int32_t max_window;           /* SF_MAX_WINDOW                                  */
} sf_model_metadata;
sf_status sortformer_get_metadata(const sf_model* model, sf_model_metadata* out);

/* Canonical tensor list (name, element count) and the fp32 value of every
 * element as generated (before any bf16 rounding); for checking the weight
 * generator. name_cap bytes are written at most (NUL-terminated). */
int32_t sortformer_num_tensors(const sf_model* model);
sf_status sortformer_tensor_info(const sf_model* model, int32_t index, char* name,
                                 int32_t name_cap, int64_t* numel);
sf_status sortformer_get_weights(const sf_model* model, int32_t index, float* host_out);

/* Host-only variants (no device needed): tensor count of a configuration,
 * and tensor `index` generated for `seed` — name (at most name_cap bytes),
 * element count and, if host_out is not NULL, its fp32 values. */
int32_t sortformer_config_num_tensors(const sf_model_config* cfg);
sf_status sortformer_config_tensor(const sf_model_config* cfg, uint64_t seed, int32_t index,
                                   char* name, int32_t name_cap, int64_t* numel,
                                   float* host_out);

/* ---------------------------------------------------------------- offline */

/* Workspace bytes for sortformer_forward_offline on `batch` clips of
 * n_samples samples each (0 if unsupported). */
size_t sortformer_offline_workspace_bytes(const sf_model* model, int32_t batch,
                                          int64_t n_samples);

/* Offline forward (NeMo SortformerEncLabelModel.forward: audio -> per-frame
 * sigmoid speaker activity).
 *  d_audio: (B, N) fp32 16 kHz mono. d_probs: (B, n_out, S) fp32 output.
 *  SORTFORMER: n_out = ceil(floor(N/160)/8) frames of 80 ms. A clip of at
 *    most SF_MAX_WINDOW encoder frames (81.9 s) is one encoder window; a
 *    longer one is processed in the 'very high' streaming configuration's
 *    chunks (340 frames + 40 look-ahead, FIFO 40, cache 188) on the
 *    known-length schedule, as the Nemotron-style variant processes its
 *    offline input in chunks; any N.
 *  NEMOTRON: the clip is processed in 30.4 s chunks with the arrival-order
 *    speaker cache and FIFO ("nemotron_offline" preset) and n_out =
 *    (8/stride)*ceil(floor(N/160)/8) frames of stride x 10 ms
 *    (SF_OPT_OUTPUT_STRIDE, default 1); any N.
 * *n_out_host receives n_out before any work is enqueued. */
sf_status sortformer_forward_offline(sf_model* model, const float* d_audio, int32_t batch,
                                     int64_t n_samples, float* d_probs, int64_t* n_out_host,
                                     void* d_workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------- streaming */

/* Device bytes of the per-stream state for `batch` lockstep streams: the
 * speaker cache, FIFO and look-ahead embeddings with their probabilities and
 * placeholder flags (NeMo API docs, SortformerStreamingState: spkcache,
 * spkcache_preds, fifo, fifo_preds and their lengths; "Streaming Sortformer
 * Diarizer" model card, Streaming Architecture), the silence statistics of
 * the placeholders, and the audio ring holding the samples the next mel
 * frames need. And the step workspace. 0 if the configuration is invalid or
 * its window (spkcache_len + fifo_len + chunk_len + right_context) exceeds
 * SF_MAX_WINDOW. */
size_t sortformer_state_bytes(const sf_model* model, const sf_stream_config* scfg,
                              int32_t batch);
size_t sortformer_stream_workspace_bytes(const sf_model* model, const sf_stream_config* scfg,
                                         int32_t batch);

/* Bind a state object to caller memory d_state (state_bytes bytes, 256-byte
 * aligned, kept alive until destroy) and reset it: the state NeMo's
 * forward_streaming_step threads through its calls (NeMo API docs,
 * SortformerStreamingState) and the Transformers streaming loop passes back
 * as speaker_cache (Transformers docs "Nemotron 3 Diarization", streaming
 * usage), here device-resident. The B streams advance in lockstep (identical
 * lengths, per-stream contents). Errors: SF_EINVAL (null pointer, invalid
 * configuration, misalignment), SF_ESHAPE (window above SF_MAX_WINDOW or
 * fewer than one cache slot per speaker), SF_ENOMEM (state too small), SF_EHIP. */
sf_status sortformer_stream_create(sf_model* model, const sf_stream_config* scfg, int32_t batch,
                                   void* d_state, size_t state_bytes, void* stream,
                                   sf_stream** out);
/* Releases the host object (waits for the device first if window graphs were
 * captured, since a replay may still be queued). */
void sortformer_stream_destroy(sf_stream* st);
/* Empty the cache/FIFO/audio history and every counter, for a new recording
 * (a runner duty the ExecuTorch issue lists in its Proposed scope, beside
 * feeding audio as it arrives and flushing the last chunk); enqueued on
 * stream. */
sf_status sortformer_stream_reset(sf_stream* st, void* stream);

/* Samples per stream the next non-final step needs (like the Transformers
 * processor's num_samples_first_audio_chunk / num_samples_per_audio_chunk):
 * step 0 needs 1280*(chunk+right_context)+40, later steps 1280*chunk. */
int64_t sortformer_stream_samples_needed(const sf_stream* st);
/* Upper bound of frames any step emits per stream (for sizing d_probs_out):
 * chunk_len + right_context for SORTFORMER, (8/stride) times that for
 * NEMOTRON (SF_OPT_OUTPUT_STRIDE of the model at the time of the call). */
int32_t sortformer_stream_max_emit(const sf_stream* st);

/* One streaming step (NeMo forward_streaming_step; Transformers model call
 * with speaker_cache): append n_new samples per stream (d_audio_new (B,
 * n_new)), compute the new mel frames and pre-encode only the new encoder
 * frames, run the encoder over [cache | FIFO | chunk | look-ahead], write the
 * chunk's probabilities to d_probs_out (B, n_emitted, S), refresh the FIFO
 * predictions, append the chunk to the FIFO, pop into the cache and compress
 * the cache when it overflows.
 * Non-final steps need n_new == sortformer_stream_samples_needed. With
 * is_last != 0 the clip ends after these n_new samples (any count >= 0): the
 * step has no look-ahead and emits every remaining frame; later steps return
 * SF_ESTATE until sortformer_stream_reset. *n_emitted_host is set before any
 * work is enqueued. No allocation and no host synchronisation. */
sf_status sortformer_stream_step(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                 int32_t is_last, float* d_probs_out, int32_t* n_emitted_host,
                                 void* d_workspace, size_t workspace_bytes, void* stream);
/* (step, continued) Errors, all returned before any work is enqueued:
 * SF_ESTATE after the final step, on a rows-only stream (set_rows), with
 * samples pending from sortformer_stream_feed, or when the counters would
 * make the step's window exceed the state's capacity; SF_ESHAPE for a wrong
 * n_new; SF_ENOMEM for a small workspace. */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as sortformer_stream_step, with its workspace taken from a static
 * device array of SF_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends, instead of a caller buffer. The
 * window forward is launched kernel by kernel (no graph capture, whose
 * instantiation may allocate), and the call makes no allocation of any kind.
 * Results are bit-identical to sortformer_stream_step's. Streams whose step
 * workspace (sortformer_stream_workspace_bytes) exceeds the scratch size get
 * SF_ENOMEM before any work; this covers a single stream of every preset but
 * "very_high" and "nemotron_offline", and small batches. All calls on one GPU
 * share its scratch array: calls that may overlap on one GPU (different host
 * threads or different HIP streams without ordering between them) race and
 * must be serialised by the caller. Other errors as sortformer_stream_step. */
#define SF_NOALLOC_SCRATCH_BYTES (64ull << 20)
sf_status sortformer_stream_step_noalloc(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                         int32_t is_last, float* d_probs_out,
                                         int32_t* n_emitted_host, void* stream);

/* Streaming feed of any sample count (the runner duties of the ExecuTorch
 * issue's Proposed scope: feed audio as it arrives, reset, flush the last
 * chunk; the Transformers streaming loop, which hands the processor audio as
 * it arrives): the n_new
 * samples per stream (d_audio_new (B, n_new)) are appended to the samples
 * already pending, every step whose audio is then complete runs exactly as
 * sortformer_stream_step would run it, and the rest stays pending in the
 * state's audio ring for the next feed. With is_last != 0 the clip ends after
 * these samples: the complete steps run, then the final step (no
 * look-ahead, every remaining frame scored). The emitted frames of all steps
 * run are written in order to d_probs_out (B, out_frames, S) at rows [0,
 * *n_emitted) of each stream (batch stride out_frames * S floats); the same
 * samples fed in any split give bit-identical outputs and state. Errors,
 * returned before any work: SF_ENOMEM if out_frames (or the workspace) is
 * too small, SF_ESTATE after the final step or on a rows-only stream. */
sf_status sortformer_stream_feed(sf_stream* st, const float* d_audio_new, int64_t n_new,
                                 int32_t is_last, float* d_probs_out, int64_t out_frames,
                                 int64_t* n_emitted_host, void* d_workspace,
                                 size_t workspace_bytes, void* stream);
/* Frames per stream a feed of n_new samples would emit now (host arithmetic;
 * -1 if the feed would be refused). */
int64_t sortformer_stream_feed_frames(const sf_stream* st, int64_t n_new, int32_t is_last);

/* State introspection for tests.
 * info (host, 9 values): cache_len, fifo_len, lookahead_len, capacity rows,
 *   steps_done, frames_emitted, samples_received, finished, samples pending
 *   (fed but not yet consumed by a step).
 * ptrs (host, 6 values): device pointers of emb (B,cap,D) fp32, probs
 *   (B,cap,S) fp32, placeholder flags (B,cap) int32, silence sum (B,D) fp64,
 *   silence count (B) int32, and the model dimension D as an integer.
 * Rows [0,cache_len) are the cache, then the FIFO, then look-ahead rows. */
sf_status sortformer_stream_get_info(const sf_stream* st, int64_t* info, void** ptrs);
/* Checkpoint / resume of the whole streaming state (NeMo API docs,
 * SortformerStreamingState, which forward_streaming_step returns and takes
 * back; the Transformers speaker_cache): cache, FIFO and look-ahead rows with
 * their probabilities and placeholder flags, the silence statistics, the
 * audio ring with any pending samples, and every counter (steps, frames
 * emitted, samples received, frames pre-encoded, finished). The blob is
 * host memory of at least sortformer_stream_checkpoint_bytes bytes, written
 * by export in a versioned layout private to this library. Import restores
 * it into any stream object of the same model architecture, speaker count,
 * batch and stream configuration (a fresh one, or the same one rewound): the
 * steps that follow are bit-identical to those of the exported stream.
 * Import checks the header (magic, version, configuration) and the counters'
 * consistency and returns SF_EINVAL with the stream untouched if either
 * fails. Both block until their copies are done. Export of a stream whose
 * rows were set by sortformer_stream_set_rows returns SF_ESTATE. */
size_t sortformer_stream_checkpoint_bytes(const sf_stream* st);
sf_status sortformer_stream_export(const sf_stream* st, void* host_blob, size_t bytes,
                                   void* stream);
sf_status sortformer_stream_import(sf_stream* st, const void* host_blob, size_t bytes,
                                   void* stream);

/* Test hooks — the rows alone: copy rows [0, cache_len + fifo_len +
 * lookahead_len) of the state to host memory (get) or from host memory (set,
 * which also sets the three lengths). Host layouts: emb (B, rows, D) fp32,
 * probs (B, rows, S) fp32, flags (B, rows) int32 (1 = silence placeholder),
 * sil_sum (B, D) fp64, sil_cnt (B) int32 (either may be NULL: not copied).
 * Both block until the copies are done. set checks the lengths against the
 * configuration (cache <= spkcache_len, fifo <= fifo_len, look-ahead <=
 * chunk_len + right_context) and leaves the step counters alone, so the
 * stream is marked rows-only: sortformer_stream_step, _feed and _export
 * return SF_ESTATE (before any work) until sortformer_stream_reset or
 * sortformer_stream_import; sortformer_stream_update is allowed. */
sf_status sortformer_stream_get_rows(const sf_stream* st, float* emb, float* probs, int32_t* flags,
                                     double* sil_sum, int32_t* sil_cnt, void* stream);
sf_status sortformer_stream_set_rows(sf_stream* st, int32_t cache_len, int32_t fifo_len,
                                     int32_t lookahead_len, const float* emb, const float* probs,
                                     const int32_t* flags, const double* sil_sum,
                                     const int32_t* sil_cnt, void* stream);

/* Stream options. SF_STREAM_OPT_GRAPHS (default 1): each step's window
 * forward (window copy + encoder + head) is captured once per distinct
 * window shape into a HIP graph on an internal stream and replayed on the
 * caller's stream; the frontend, pre_encode and the cache update stay
 * direct launches. 0 launches every kernel directly. Results are identical
 * either way. Graphs are kept for one workspace pointer at a time (at most two
 * per window size): a step with another workspace, or turning the option
 * off, first waits for the device once and releases the old graphs; steps
 * with an unchanged workspace never synchronise the host. */
#define SF_STREAM_OPT_GRAPHS 1
/* SF_STREAM_OPT_FIXED_WINDOW (default 0): with 1 every step's window forward
 * runs at one fixed size, the stream's capacity (spkcache_len + fifo_len +
 * chunk_len + right_context rows), with the rows past the current window
 * zeroed and masked: the valid length is written to the workspace by a small
 * kernel before each window forward and every kernel that masks reads it
 * there. One graph per ping-pong buffer then serves every step (the
 * Transformers docs "Nemotron 3 Diarization", fixed-window section: pad to
 * max_window so that one compiled graph serves the whole stream), at the cost
 * of computing the padded rows. Valid rows are unchanged by the padding
 * (bit for bit while the padded and unpadded windows fall on the same side
 * of the 4096-row kernel regimes). */
#define SF_STREAM_OPT_FIXED_WINDOW 2
sf_status sortformer_stream_set_option(sf_stream* st, int32_t option, int32_t value);

/* Test hook — the cache update alone ("Streaming Sortformer Diarizer" model
 * card, Streaming Architecture: FIFO prediction refresh, chunk append, pop
 * with silence statistics, compression), given window probabilities
 * d_window_probs (B, W, S) with W = cache_len + fifo_len + lookahead_len of
 * the current state; the first n_chunk look-ahead rows are the chunk. */
sf_status sortformer_stream_update(sf_stream* st, const float* d_window_probs, int32_t n_chunk,
                                   void* d_workspace, size_t workspace_bytes, void* stream);

/* Test hook — the encoder alone on explicit window embeddings: d_emb (B, W,
 * 512) fp32 pre-encoded frames, rows >= n_valid are right padding (masked
 * keys, zeroed conv input). Writes d_probs (B, W, S) at 80 ms and, for
 * NEMOTRON, d_probs10 (B, 8W, S) (may be NULL for SORTFORMER). */
size_t sortformer_encode_workspace_bytes(const sf_model* model, int32_t batch, int32_t window);
sf_status sortformer_encode_window(sf_model* model, const float* d_emb, int32_t batch,
                                   int32_t window, int32_t n_valid, float* d_probs,
                                   float* d_probs10, void* d_workspace, size_t workspace_bytes,
                                   void* stream);

/* Test hook — per-layer taps for sortformer_encode_window ("Streaming
 * Sortformer Diarizer" model card, Pipeline: the FastConformer and
 * Transformer layers; Nemotron card summary: the RoPE layers). While a tap
 * (layer, point) is registered, every sortformer_encode_window call on the
 * model also writes that activation, widened to fp32, as (B, W, d)
 * row-major into d_out, for all W rows (rows >= n_valid hold whatever the
 * padded computation produced). Layers: SORTFORMER 0..16 are the conformer
 * layers (d 512) and 17..34 the transformer layers (d 192); NEMOTRON 0..30
 * (d 512). d_out is a device buffer of out_floats floats owned by the
 * caller, which must keep it alive while the tap is registered; an
 * encode_window call whose taps need more than out_floats returns SF_ENOMEM
 * and enqueues nothing. d_out NULL removes the (layer, point) tap; layer -1
 * with d_out NULL removes all. At most SF_MAX_TAPS taps; registering an
 * existing (layer, point) replaces its buffer. Not thread-safe with calls on
 * the same model; the offline and streaming calls ignore taps.
 * Returns SF_EINVAL (null model, bad point, too many taps) or SF_ESHAPE
 * (layer out of range). */
#define SF_TAP_LAYER_IN 0  /* residual stream entering the layer, fp32              */
#define SF_TAP_ATTN_CTX 1  /* attention context of all heads before W_o (compute    */
                           /* dtype, widened)                                       */
#define SF_TAP_LAYER_OUT 2 /* layer output as the next stage reads it: the fp32     */
                           /* residual stream, except conformer layer 16 (the       */
                           /* compute-dtype LN_out output fed to encoder_proj) and  */
                           /* NEMOTRON layer 30 (after the final LayerNorm)         */
#define SF_MAX_TAPS 16
sf_status sortformer_debug_tap(sf_model* model, int32_t layer, int32_t point, float* d_out,
                               size_t out_floats);

/* Test hook — frontend and pre_encode alone: d_audio (B, N) -> d_mel (B, T,
 * 128) with T = floor(N/160), and -> d_emb (B, ceil(T/8), 512). Either
 * output may be NULL. Workspace: sortformer_pre_encode_workspace_bytes. */
size_t sortformer_pre_encode_workspace_bytes(const sf_model* model, int32_t batch,
                                             int64_t n_samples);
sf_status sortformer_pre_encode(sf_model* model, const float* d_audio, int32_t batch,
                                int64_t n_samples, float* d_mel, float* d_emb,
                                void* d_workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ segments */

/* Speaker-activity probabilities -> speech segments. The pages give the
 * output of diarization as [begin_seconds, end_seconds, speaker_index]
 * segments obtained by VAD-style thresholding and smoothing of the sigmoid
 * probabilities ("Streaming Sortformer Diarizer" model card, Output; NeMo API
 * docs, diarize() Returns; Transformers docs, extract_speaker_dict). The
 * parameters and their order are not printed there; per (stream, speaker)
 * track this library applies, in order:
 *  1. hysteresis in fp32: on when p > onset, off when p <= offset, else the
 *     previous frame's state (off before the first frame); onset >= offset;
 *  2. each maximal run of "on" frames [f0, f1) -> [f0*frame_s, f1*frame_s];
 *  3. start -= pad_onset, end += pad_offset, clipped to [0, T*frame_s];
 *  4. a segment whose gap to the previous one is below min_duration_off is
 *     merged into it (overlaps always merge);
 *  5. segments shorter than min_duration_on are dropped.
 * Times are computed in fp64. Defaults: onset = offset = 0.5, everything else
 * 0 (the segments are then exactly the runs of frames with p > 0.5). */
typedef struct sf_segment_params {
  float onset, offset;
  double pad_onset, pad_offset;
  double min_duration_on, min_duration_off;
} sf_segment_params;

typedef struct sf_segment {
  double start_s, end_s;
  int32_t speaker, stream;
} sf_segment;

void sortformer_segment_defaults(sf_segment_params* out);
/* Most segments one track can hold: (T + 1) / 2. */
int64_t sortformer_segments_capacity(int64_t n_frames);
/* d_probs (B, T, S) fp32 on the device (S <= 64, frame_s > 0). Writes track
 * (b, s)'s segments in time order to d_out[(b*S + s)*capacity ...] and their
 * number to d_counts[b*S + s] (int64). capacity must be at least
 * sortformer_segments_capacity(T) (SF_ENOMEM otherwise); params NULL = the
 * defaults; invalid parameters -> SF_EINVAL. */
sf_status sortformer_segments(const float* d_probs, int32_t batch, int64_t n_frames,
                              int32_t n_spk, double frame_s, const sf_segment_params* params,
                              sf_segment* d_out, int64_t capacity, int64_t* d_counts,
                              void* stream);

/* --------------------------------------------------------------- profiling */

/* Benchmark aid: while a kernel class is profiled, every launch of that
 * class is bracketed by a pair of HIP events recorded on the launch's stream,
 * and the launch's algorithmic flop and byte counts are added up (what the
 * operation must compute and move). One class at a time; at most
 * max_launches launches are timed. Not thread-safe. */
#define SF_PROF_GEMM 1
#define SF_PROF_ATTN 2
#define SF_PROF_LN 3
#define SF_PROF_CONV 4
#define SF_PROF_FRONTEND 5
#define SF_PROF_CACHE 6
sf_status sortformer_profile_begin(int32_t kernel_class, int32_t max_launches);
/* Waits for the recorded events; returns the summed kernel time (ms), the
 * launch count and the algorithmic flops and bytes of those launches. */
sf_status sortformer_profile_end(double* total_ms, int64_t* launches, double* flops,
                                 double* bytes);

#ifdef __cplusplus
}
#endif
#endif /* SORTFORMER_H */
