/*
 * dart.h - C ABI of the DART hot path on AMD Instinct MI355X (gfx950).
 *
 * DART ("Decoded Attention over Recurrent sTates") keeps the per-chunk state
 * contributions of the Mamba-2 chunked scan as chunk memories dH[c] (N x P),
 * decodes a token-conditioned key dH[c]·E_t and value C_tᵀ·dH[c] from each,
 * runs softmax attention (state-memory attention, SMA) over the completed
 * chunks with query Q_t, and adds the readout to the Mamba-2 output through
 * a scalar gate.  Sources: DART abstract (aipentium and mlsanity pages); Pith
 * review of DART, "Core claim", "What carries the argument", referee major
 * comment 3 (paper §3 Eq. 8) and minor comment 1 (paper §4 Eq. 14).
 *
 * Prefill is three calls on one stream, in this order:
 *   dart_chunk_scan -> dart_chunk_out -> dart_sma_fwd
 * (or, with the f32 memories kept as an output and the state recurrence as a
 * pass of its own: dart_chunk_state -> dart_state_pass -> dart_sma_fwd).
 * Decode is one call per generated token: dart_sma_decode.
 * Extensions of the same path:
 *   training: dart_sma_fwd_train in place of dart_sma_fwd, then the backward
 *             dart_sma_bwd -> dart_scan_bwd (its memory gradient and the SMA
 *             part of dC feed the scan backward);
 *   the decay-included SMA variant: dart_sma_fwd_decayed;
 *   chunked prefill from a decode cache: dart_sma_fwd_cont (with h0 given to
 *             dart_state_pass);
 *   an fp8 chunk-memory cache: dart_cache_fp8_store, dart_sma_decode_fp8,
 *             dart_sma_fwd_cont_fp8.
 *
 * Conventions for every call
 * --------------------------
 * - Every tensor argument is a pointer to DEVICE memory owned by the caller,
 *   dense row-major in the layout given, 16-byte aligned.  The library never
 *   allocates, frees or keeps memory, and holds no global state, apart from
 *   the static device scratch of dart_sma_decode_noalloc and a call counter
 *   that tags dart_chunk_scan's workspace flags.
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work and return; results are ready once the stream reaches them.
 * - Dimensions and pointers are validated on the host before any HIP call; a
 *   non-OK status means nothing was enqueued.  DART_ERR_HIP reports a launch
 *   failure; a fault inside a kernel surfaces at the caller's next
 *   synchronisation.
 * - Outputs never alias inputs (decode state arguments are in/out; the one
 *   documented exception is dart_scan_bwd's dC_sma, which may be dC).
 * - Symbols: B batch, L sequence length, H heads, G groups (B, C and Q are
 *   shared by H/G consecutive heads), N state size (key axis), P head dim
 *   (value axis), S chunk size, M = L/S chunks, k = floor(t/S) the chunk of
 *   token t.  "io" is the element type named by dart_dims.io.
 * - State matrices (dH, H_in, h0, decode cache, h, dH_cur) are N x P
 *   matrices stored value-axis-major: element (n, p) sits at [p][n], i.e.
 *   the key axis N is contiguous.
 *
 * Supported shapes: io = DART_F32 with (N, P) in {(16,16), (32,32)};
 * io = DART_BF16 with (N, P) in {(32,32), (64,64), (128,64), (128,128)};
 * S a multiple of 32 with 32 <= S <= 256; L a multiple of S.  Anything else
 * returns DART_ERR_UNSUPPORTED (shape) or DART_ERR_BAD_DIMS (inconsistent).
 */
#ifndef DART_H
#define DART_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dart_status {
  DART_OK = 0,
  DART_ERR_NULL_PTR = 1,    /* a required pointer is NULL                   */
  DART_ERR_BAD_DIMS = 2,    /* non-positive dim, L % S != 0, H % G != 0 ... */
  DART_ERR_UNSUPPORTED = 3, /* (dtype, N, P, S) outside the compiled set    */
  DART_ERR_DTYPE = 4,       /* io is not a dart_dtype value                 */
  DART_ERR_WORKSPACE = 5,   /* decode workspace missing or too small        */
  DART_ERR_HIP = 6,         /* a HIP launch reported an error               */
  DART_ERR_ALIGN = 7,       /* a pointer is not 16-byte aligned             */
  DART_ERR_SCRATCH = 8      /* dims exceed the static scratch of the
                               allocation-free decode entry point           */
} dart_status;

typedef enum dart_dtype { DART_F32 = 0, DART_BF16 = 1 } dart_dtype;

/* Prefill dimensions. */
typedef struct dart_dims {
  int64_t batch, seqlen, nheads, ngroups, dstate /* N */, headdim /* P */, chunk /* S */;
  int32_t io; /* dart_dtype of x, Bm, C, Q, E, dH and y */
} dart_dims;

/* Decode dimensions; max_chunks is the cache capacity per (sequence, head). */
typedef struct dart_decode_dims {
  int64_t batch, nheads, ngroups, dstate, headdim, chunk, max_chunks;
  int32_t io; /* dart_dtype of x, Bm, C, Q, E, cache and y */
} dart_decode_dims;

/*
 * Chunk state memories (first step of the Mamba-2 chunked scan).
 * Source: Pith review of DART, "What carries the argument" (dH[c] is the
 * N x P contribution of chunk c to the chunk-boundary state) and the axiom
 * ledger (the chunked scan yields these contributions).
 *
 *   acum[b,h,c,s] = sum_{j<=s} dt[b,cS+j,h]·A[h]            (inclusive)
 *   dH[b,h,c]     = sum_{i in c} exp(acum_end - acum_i)·dt_i·B_i x_iᵀ
 *
 * in:  x [B,L,H,P] io; dt [B,L,H] f32 (> 0); A [H] f32 (< 0);
 *      Bm [B,L,G,N] io
 * out: acum [B,H,M,S] f32; dH [B,H,M,P,N] io (rounded to nearest even);
 *      dH_f32 [B,H,M,P,N] f32 (the same memories unrounded, for the state
 *      recurrence).
 */
dart_status dart_chunk_state(const dart_dims* dims, const void* x, const float* dt,
                             const float* A, const void* Bm, float* acum, void* dH,
                             float* dH_f32, void* stream);

/*
 * Inter-chunk state passing and the native Mamba-2 output y_ssd.
 * Source: Pith review of DART, axiom ledger (SSD as structured causal
 * attention, paper Eq. 4; intra- and inter-chunk terms of the chunked scan)
 * and "Core claim" (Mamba-2 reads values from its state as C_t·H_t).
 *
 *   H[0] = h0 (zero when h0 == NULL)
 *   H[c+1] = exp(acum[c, S-1])·H[c] + dH_f32[c]      (recurrence in f32)
 *   H_in[c] = io(H[c]) for c < M;  h_final = H[M]
 *   y_ssd[t] = sum_{j in k, j<=t} (C_t·B_j)·exp(acum_t - acum_j)·dt_j·x_j
 *            + exp(acum_t)·C_tᵀ·H_in[k]
 *
 * in:  x, dt, Bm as above; C [B,L,G,N] io; acum, dH_f32 from
 *      dart_chunk_state; h0 [B,H,P,N] f32 or NULL
 * out: H_in [B,H,M,P,N] io, the state entering each chunk, rounded to the io
 *      type once (the precision y_ssd's inter-chunk product uses);
 *      h_final [B,H,P,N] f32, the state after the last chunk (the decode
 *      state h that continues this sequence); y_ssd [B,L,H,P] io (rounded
 *      to the io type once, like every io-typed output)
 */
dart_status dart_state_pass(const dart_dims* dims, const void* x, const float* dt,
                            const void* Bm, const void* C, const float* acum,
                            const float* dH_f32, const float* h0, void* H_in,
                            float* h_final, void* y_ssd, void* stream);

/*
 * Chunk memories and the inter-chunk state recurrence in one pass: the
 * outputs of dart_chunk_state and the state half of dart_state_pass
 * without the f32 memories round trip through memory.
 * Source: as dart_chunk_state and dart_state_pass (Pith review of DART, axiom
 * ledger: the chunked scan's chunk contributions and inter-chunk state
 * passing; "What carries the argument": dH[c] is chunk c's contribution to
 * the chunk-boundary state).
 *
 *   acum, dH            as dart_chunk_state
 *   H[0] = h0 (zero when h0 == NULL)
 *   H[c+1] = exp(acum[c, S-1])·H[c] + dH_f32[c]     (f32, in chunk order)
 *   H_in[c] = io(H[c]) for c < M;  h_final = H[M]
 * The results are bit-identical to dart_chunk_state followed by
 * dart_state_pass.
 *
 * in:  x [B,L,H,P] io; dt [B,L,H] f32; A [H] f32; Bm [B,L,G,N] io;
 *      h0 [B,H,P,N] f32 or NULL
 * out: acum [B,H,M,S] f32; dH [B,H,M,P,N] io; dH_f32 [B,H,M,P,N] f32 when
 *      not NULL (the unrounded memories; NULL skips them); H_in [B,H,M,P,N]
 *      io; h_final [B,H,P,N] f32
 * workspace: device memory of at least dart_chunk_scan_workspace(dims) bytes
 *      (workspace_bytes gives its size; smaller returns DART_ERR_WORKSPACE).
 *      Any initial contents.  For 16-bit io it holds one f32 state slot pair
 *      and one flag per (batch, head), through which the workgroup of each
 *      group of chunks hands its outgoing state to the next; each call tags
 *      its flags with a per-call number, so a flag left by an earlier call
 *      never passes for this one.  Every wait is bounded: a wait that gives
 *      up (which a correct launch never does) adds one to the workspace's
 *      first int32 and leaves that call's outputs undefined; callers that
 *      check it zero that int32 beforehand.  Calls that share a workspace
 *      must not overlap (the same stream, or ordered streams).  For f32 io
 *      the workspace holds the f32 memories of a two-pass recurrence.
 */
size_t dart_chunk_scan_workspace(const dart_dims* dims);
dart_status dart_chunk_scan(const dart_dims* dims, const void* x, const float* dt,
                            const float* A, const void* Bm, const float* h0, float* acum,
                            void* dH, float* dH_f32, void* H_in, float* h_final,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The native Mamba-2 chunk output alone (the y_ssd half of dart_state_pass),
 * from H_in as dart_chunk_scan or dart_state_pass wrote it.
 * Source: Pith review of DART, axiom ledger (SSD as structured causal
 * attention, paper Eq. 4; intra- and inter-chunk terms of the chunked scan)
 * and "Core claim" (Mamba-2 reads values from its state as C_t·H_t).
 *
 *   y_ssd[t] = sum_{j in k, j<=t} (C_t·B_j)·exp(acum_t - acum_j)·dt_j·x_j
 *            + exp(acum_t)·C_tᵀ·H_in[k]
 *
 * in:  x, dt, Bm as dart_chunk_state; C [B,L,G,N] io; acum [B,H,M,S] f32;
 *      H_in [B,H,M,P,N] io
 * out: y_ssd [B,L,H,P] io (bit-identical to dart_state_pass's)
 */
dart_status dart_chunk_out(const dart_dims* dims, const void* x, const float* dt,
                           const void* Bm, const void* C, const float* acum, const void* H_in,
                           void* y_ssd, void* stream);

/*
 * State-memory attention over completed chunks plus the gated add.
 * Source: Pith review of DART, "Core claim" and "What carries the argument"
 * (key dH[c]·E_t, value C_tᵀ·dH[c], query Q_t, scalar gate), referee major
 * comment 3 (paper §3 Eq. 8: raw memories, no decay); DART abstract.
 *
 *   s[t,c] = Q_tᵀ·dH[c]·E_t / sqrt(N)          for c < k (k = chunk of t)
 *   o_t    = sum_{c<k} softmax_c(s[t,c])·C_tᵀ·dH[c]   (o_t = 0 when k = 0)
 *   y_t    = y_ssd_t + gate·o_t
 *
 * in:  Q [B,L,G,N] io; E [B,L,H,P] io; C [B,L,G,N] io; dH [B,H,M,P,N] io;
 *      y_ssd [B,L,H,P] io (as written by dart_state_pass)
 * out: y [B,L,H,P] io
 */
dart_status dart_sma_fwd(const dart_dims* dims, const void* Q, const void* E,
                         const void* C, const void* dH, const void* y_ssd, float gate,
                         void* y, void* stream);

/*
 * Continuation of sequences that already hold prior_chunks completed chunks
 * (chunked prefill after an earlier prefill or decode).  The L = M·S tokens
 * of dims are chunks prior_chunks .. prior_chunks+M-1 of their sequences;
 * their memories dH come from dart_chunk_state on these tokens and their
 * y_ssd from dart_state_pass with h0 = the state after the prior chunks.
 * Token t of local chunk j attends to memories c < prior_chunks + j:
 * memory c < prior_chunks is cache[b,h,c], memory prior_chunks + i is
 * dH[b,h,i]; otherwise the formulas of dart_sma_fwd.  prior_chunks = 0 is
 * dart_sma_fwd.
 *
 * in:  Q, E, C, dH, y_ssd as dart_sma_fwd; cache [B,H,cache_chunks,P,N] io
 *      (the dart_sma_decode cache layout; may be NULL when prior_chunks = 0)
 * out: y [B,L,H,P] io
 * errors: DART_ERR_BAD_DIMS unless 0 <= prior_chunks <= cache_chunks
 */
dart_status dart_sma_fwd_cont(const dart_dims* dims, int64_t prior_chunks, int64_t cache_chunks,
                              const void* Q, const void* E, const void* C, const void* cache,
                              const void* dH, const void* y_ssd, float gate, void* y,
                              void* stream);

/*
 * The decay-included variant of dart_sma_fwd, the ablation the Pith review
 * of DART asks for (referee major comment 3, paper §3 Eq. 8): key and value
 * of memory c are scaled, for token t of chunk k > c, by the decay the SSM
 * applies between the end of chunk c and t,
 *
 *   d[t,c] = exp(sum_{j = end(c)+1 .. t} dt_j·A) = exp(acum[k, t-kS] + sum_{c<c'<k} acum[c', S-1])
 *   s[t,c] = d[t,c]·Q_tᵀ·dH[c]·E_t / sqrt(N),
 *   o_t    = sum_{c<k} softmax_c(s[t,c])·d[t,c]·C_tᵀ·dH[c],   y_t = y_ssd_t + gate·o_t
 *
 * in:  as dart_sma_fwd, plus acum [B,H,M,S] f32 from dart_chunk_state
 * out: y [B,L,H,P] io
 */
dart_status dart_sma_fwd_decayed(const dart_dims* dims, const void* Q, const void* E,
                                 const void* C, const void* dH, const float* acum,
                                 const void* y_ssd, float gate, void* y, void* stream);

/*
 * Training forward of SMA: dart_sma_fwd plus the statistics the backward
 * reads.  Same formulas and arguments as dart_sma_fwd, and
 * out: o [B,L,H,P] f32, the readout before the gate (0 for chunk-0 tokens);
 *      lse [B,H,L] f32, the softmax log-normaliser of each token in base-2
 *      units of the scaled score, log2 Σ_c 2^(s_{t,c}·log2(e)) (0 for
 *      chunk-0 tokens).
 */
dart_status dart_sma_fwd_train(const dart_dims* dims, const void* Q, const void* E,
                               const void* C, const void* dH, const void* y_ssd, float gate,
                               void* y, void* o, float* lse, void* stream);

/*
 * Backward of SMA and the gated add (the reverse-mode derivative of
 * dart_sma_fwd; Pith review of DART, "Core claim": the path is trained end
 * to end).  With do_t = gate·dy_t, α the softmax weights (recomputed from
 * lse) and D_t = do_t·o_t, for token t of chunk k and memory c < k:
 *   ds      = α·(do_t·(C_tᵀ·dH[c]) − D_t)
 *   dE_t    = Σ_c ds·dH[c]ᵀ·Q_t / sqrt(N)
 *   dQ_t    = Σ_c ds·dH[c]·E_t / sqrt(N)      (summed over the group's heads)
 *   dC_t    = Σ_c α·dH[c]·do_t                (SMA part; summed likewise)
 *   ddH[c]  = Σ_t ds·Q_t E_tᵀ / sqrt(N) + α·C_t do_tᵀ
 *   dgate   = Σ dy·o;   the gradient of y_ssd is dy itself (not written).
 * in:  Q, C [B,L,G,N], E [B,L,H,P], dH [B,H,M,P,N] (io), o [B,L,H,P] f32 and
 *      lse [B,H,L] f32 (both from dart_sma_fwd_train), dy [B,L,H,P] io, gate
 * out: dQ, dC [B,L,G,N] f32; dE [B,L,H,P] f32; ddH [B,H,M,P,N] f32;
 *      dgate: one f32 (device memory)
 * workspace: device memory of at least dart_sma_bwd_workspace(dims) bytes:
 *      about 4·B·H·L bytes plus 8 bytes per visible (token, memory) pair,
 *      B·H·L·(M-1)/2 of them (~130 MB at B=4, H=32, L=8192, S=256).
 * Compiled for bf16 io with P <= 64 and chunks that are multiples of 64
 * (MFMA kernels), and for every f32 io shape and chunk size (plain f32
 * kernels, the f32 correctness shapes); other dims return
 * DART_ERR_UNSUPPORTED.
 */
size_t dart_sma_bwd_workspace(const dart_dims* dims);
dart_status dart_sma_bwd(const dart_dims* dims, const void* Q, const void* E, const void* C,
                         const void* dH, const void* o, const float* lse, const void* dy,
                         float gate, float* dQ, float* dE, float* dC, float* ddH, float* dgate,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the chunked scan (dart_chunk_state + dart_state_pass; the
 * Mamba-2 SSD that the Pith review's axiom ledger and "What carries the
 * argument" describe).  With u_t = acum (the log-decay from the start of
 * token t's chunk) and U_c its value at the chunk's last token:
 *   dH[c]      = Σ_i exp(U_c − u_i)·dt_i·B_i x_iᵀ
 *   H_in[c+1]  = exp(U_c)·H_in[c] + dH[c]
 *   y_ssd_t    = Σ_{j<=t} (C_t·B_j)·exp(u_t − u_j)·dt_j·x_j + exp(u_t)·C_tᵀH_in[k]
 * and the upstream gradients dy (of y_ssd; the gated add passes dy through
 * unchanged), ddH (of the memories, e.g. from dart_sma_bwd; may be NULL)
 * and dh_final (of the final state; may be NULL), this returns the
 * gradients of x, dt, A, B, C and of the initial state.
 * in:  x, dy [B,L,H,P] io; dt [B,L,H] f32; A [H] f32; Bm, C [B,L,G,N] io;
 *      acum [B,H,M,S] f32 (dart_chunk_state); H_in [B,H,M,P,N] io
 *      (dart_state_pass); ddH [B,H,M,P,N] f32; dh_final [B,H,P,N] f32;
 *      dC_sma [B,L,G,N] f32 or NULL: added to dC (dC_sma may be dC itself)
 * out: dx [B,L,H,P], ddt [B,L,H], dA [H], dB, dC [B,L,G,N], dh0 [B,H,P,N],
 *      all f32 (dB and dC summed over the heads of each group)
 * workspace: at least dart_scan_bwd_workspace(dims) bytes of device memory.
 * Compiled for bf16 io with P <= 64 and chunks that are multiples of 64
 * (MFMA kernels), and for every f32 io shape and chunk size (plain f32
 * kernels); other dims return DART_ERR_UNSUPPORTED.
 */
size_t dart_scan_bwd_workspace(const dart_dims* dims);
dart_status dart_scan_bwd(const dart_dims* dims, const void* x, const float* dt, const float* A,
                          const void* Bm, const void* C, const float* acum, const void* H_in,
                          const void* dy, const float* ddH, const float* dh_final,
                          const float* dC_sma, float* dx, float* ddt, float* dA, float* dB,
                          float* dC, float* dh0, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of device workspace dart_sma_decode needs for these dims (a
 * multiple of 256; 0 if the dims are invalid). */
size_t dart_sma_decode_workspace(const dart_decode_dims* dims);

/*
 * One decode step: one new token per sequence over the chunk-memory cache.
 * Source: DART abstract (the length-dependent inference cache is the set of
 * chunk memories); Pith review minor comment 1 (paper §4 Eq. 14).
 *
 * For each (b, h), with k = n_chunks[b] and the token at position pos[b] of
 * chunk k:
 *   1. a = exp(dt·A); h <- a·h + dt·B xᵀ; dH_cur <- a·dH_cur + dt·B xᵀ;
 *      y_ssd = Cᵀ·h
 *   2. o = SMA over cache[0..k-1] with the dart_sma_fwd formulas
 *   3. y = y_ssd + gate·o
 *   4. if pos[b] == S-1: cache[k] <- io(dH_cur), dH_cur <- 0,
 *      n_chunks[b] += 1, pos[b] <- 0; else pos[b] += 1.
 *
 * in:     x [B,H,P] io; dt [B,H] f32; A [H] f32; Bm, C, Q [B,G,N] io;
 *         E [B,H,P] io
 * in/out: cache [B,H,max_chunks,P,N] io; h, dH_cur [B,H,P,N] f32;
 *         n_chunks [B] int32; pos [B] int32 (all device memory)
 * out:    y [B,H,P] io
 * workspace: device memory of at least dart_sma_decode_workspace(dims)
 *         bytes; its first int32 is set to 1 (never cleared by the library)
 *         when a chunk could not be appended because n_chunks[b] had reached
 *         max_chunks (the cache is never written out of bounds; n_chunks
 *         then stays at max_chunks).  One workspace serves one call at a time.
 */
dart_status dart_sma_decode(const dart_decode_dims* dims, const void* x, const float* dt,
                            const float* A, const void* Bm, const void* C, const void* Q,
                            const void* E, float gate, void* cache, float* h,
                            float* dH_cur, int32_t* n_chunks, int32_t* pos, void* y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of dart_sma_decode, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * steps and results as dart_sma_decode, except:
 * - no workspace: the y_ssd rows and per-split partials live in a static
 *   device array of DART_DECODE_SCRATCH_BYTES per GPU, which the library
 *   holds from its first use on that GPU until the process ends.  Dims whose
 *   dart_sma_decode_workspace() exceeds that size return DART_ERR_SCRATCH
 *   (at N = 128, P = 64: beyond about 8,000 (sequence, head) pairs).  Nothing
 *   in it needs clearing between calls (every call writes what it reads).
 * - cache_full: a caller-owned device int32 (4-byte aligned), or NULL; set
 *   to 1 (never cleared) when a chunk could not be appended because
 *   n_chunks[b] had reached max_chunks (the workspace flag of
 *   dart_sma_decode).  With NULL the condition is not reported.
 * The function calls no allocator.  Its first call on a device looks up the
 * array's address with that device current.  All calls on one GPU share the
 * one array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.
 */
#define DART_DECODE_SCRATCH_BYTES (4u << 20)
dart_status dart_sma_decode_noalloc(const dart_decode_dims* dims, const void* x,
                                    const float* dt, const float* A, const void* Bm,
                                    const void* C, const void* Q, const void* E, float gate,
                                    void* cache, float* h, float* dH_cur, int32_t* n_chunks,
                                    int32_t* pos, void* y, int32_t* cache_full, void* stream);

/*
 * fp8 chunk-memory cache.  Source: Pith review of DART, "Where Pith is
 * reading between the lines" (editorial extensions: because SMA reads the
 * chunked scan's own dH, the memory cache can be combined with cache
 * quantisation).  The pages fix no format; this library's format is:
 *
 *   cache8 [B,H,max_chunks,P,N] uint8: OCP FP8 E4M3 codes (sign, 4 exponent
 *          bits with bias 7, 3 mantissa bits; no infinities, 0x7F and 0xFF
 *          are NaN, largest finite value 448), in the layout of the io cache
 *   scale  [B,H,max_chunks] f32: one power-of-two scale per memory
 *
 * Memory c of (b, h) stands for decode(cache8[b,h,c])·scale[b,h,c].  For a
 * memory M with largest magnitude amax = f·2^E (0.5 <= f < 1) the scale is
 * 2^e with e = max(E - 8, -126) (1 when amax = 0), and each code is M·2^-e
 * rounded to the nearest E4M3 value, ties to even mantissa; |M·2^-e| < 256,
 * so no code saturates.  The memories must be finite.
 */

/*
 * Encode f32 memories into fp8 cache slots: for each (b, h) and i < n_mem,
 * memory dH_f32[b,h,i] goes to slot first + i (codes and scale as above).
 * Used after a prefill (dH_f32 of dart_chunk_state) to fill the cache that
 * dart_sma_decode_fp8 reads.
 *
 * dims:   the decode dims of the cache (batch, nheads, dstate N, headdim P,
 *         max_chunks, io; ngroups and chunk are validated but unused)
 * in:     dH_f32 [B,H,n_mem,P,N] f32
 * out:    cache8 slots [first, first + n_mem) and their scales
 * errors: DART_ERR_BAD_DIMS unless 0 <= n_mem and 0 <= first <= max_chunks
 *         - n_mem; n_mem = 0 writes nothing.
 */
dart_status dart_cache_fp8_store(const dart_decode_dims* dims, const float* dH_f32,
                                 int64_t n_mem, int64_t first, uint8_t* cache8, float* scale,
                                 void* stream);

/*
 * dart_sma_decode over the fp8 cache: identical steps and arguments except
 * that the cache is (cache8, scale) in the format above.  Step 2 reads the
 * memories decode(code)·scale; step 4 appends dH_cur (f32) encoded with its
 * own scale.  Workspace: dart_sma_decode_workspace(dims) bytes, as for
 * dart_sma_decode.
 */
dart_status dart_sma_decode_fp8(const dart_decode_dims* dims, const void* x, const float* dt,
                                const float* A, const void* Bm, const void* C, const void* Q,
                                const void* E, float gate, uint8_t* cache8, float* scale,
                                float* h, float* dH_cur, int32_t* n_chunks, int32_t* pos, void* y,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * dart_sma_fwd_cont over the fp8 cache: identical steps and arguments except
 * that prior memory c < prior_chunks of (b, h) is decode(cache8[b,h,c])·
 * scale[b,h,c] (the format above; cache8 [B,H,cache_chunks,P,N],
 * scale [B,H,cache_chunks]).  The product is taken in bfloat16, where it is
 * exact for memories of normal magnitude.  io must be DART_BF16.
 *
 * errors: DART_ERR_UNSUPPORTED for io = DART_F32; DART_ERR_BAD_DIMS unless
 *         0 <= prior_chunks <= cache_chunks; cache8 and scale may be NULL
 *         when prior_chunks = 0.
 */
dart_status dart_sma_fwd_cont_fp8(const dart_dims* dims, int64_t prior_chunks,
                                  int64_t cache_chunks, const void* Q, const void* E,
                                  const void* C, const uint8_t* cache8, const float* scale,
                                  const void* dH, const void* y_ssd, float gate, void* y,
                                  void* stream);

/* Host-only checks (no HIP call; usable without a GPU). */
dart_status dart_validate_dims(const dart_dims* dims);
dart_status dart_validate_decode_dims(const dart_decode_dims* dims);

/* Static, human-readable name of a status. */
const char* dart_status_str(dart_status status);

#ifdef __cplusplus
}
#endif

#endif /* DART_H */
