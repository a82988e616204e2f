/*
 * libsinkroute: sink-aware routed GQA decode attention for MI355X (gfx950).
 *
 * One decode step of one attention layer, single query token per sequence:
 *
 *   sr_record_sink   prefill side: keep the key and value at position 0.
 *   sr_route         score every query head against the position-0 key,
 *                    decide per KV group (sink / active) and emit a compacted
 *                    work list, all on the device.
 *   sr_decode_attn   sink groups write the position-0 value; active groups run
 *                    split-K flash-decode with an fp32 online softmax, merged
 *                    in-kernel by the last workgroup to finish an item.
 *   sr_dense_decode  the same kernel with routing off (every group active).
 *
 * The method is SinkRouter as described by its GitHub README
 * (github.com/streamer-AP/SinkRouter, the list of decode-time steps and the
 * routing-controls section) and by the pith.science rendering of the paper
 * (arXiv 2604.16883: Eq. (1) in the Figure 1 caption, the Figure 4 workflow,
 * the Figure 10 KV-group cosine proxy).
 *
 * Conventions shared by every call
 * --------------------------------
 *  B  batch, Hq query heads, Hkv KV heads, G = Hq / Hkv, d head dim,
 *  T  cached positions 0..T-1 (all of them are attended; the caller has
 *     already appended the current token's key and value).
 *  Item j = b * Hkv + g is one (sequence, KV group) pair; query head h belongs
 *  to group h / G (Hugging Face repeat_kv layout).
 *
 *  Caches k_cache / v_cache: element (b, g, t, i) lives at
 *     base + b*stride_b + g*stride_h + t*stride_t + i        (in elements)
 *  so d is contiguous and T_max >= T is allowed.  Element type is bf16 or
 *  fp32 (kv_dtype).  Every row start must be 16-byte aligned.
 *  q, out: fp32 [B][Hq][d] contiguous.  k0, v0: fp32 [B][Hkv][d] contiguous.
 *  q, out and k0 are read or written 16 bytes at a time and must start
 *  16-byte aligned; the other arrays need their element's alignment.  out
 *  must not overlap q (SR_ERR_INVALID_ARG): workgroups still read q while
 *  others write their rows of out.
 *
 *  Pointers: every data pointer is a device pointer owned by the caller; the
 *  library never allocates, frees or keeps them.  `stream` is a hipStream_t
 *  (NULL = the default stream).  Calls only enqueue work: none of them waits
 *  for the device, so results are ready once the stream is synchronised.
 *  The only state the library keeps is the CU count of each device it meets
 *  and, for sr_route_decode_static only, one scratch array per device.
 *
 *  Errors: arguments are checked on the host before anything is enqueued, so
 *  a call that returns an error has done nothing.  SR_ERR_UNSUPPORTED means
 *  the shape is outside the envelope below (the caller should use its
 *  standard attention path, as the README's routing-controls section does
 *  for shapes its kernel does not cover).  SR_ERR_HIP reports a failed launch.
 *
 *  Envelope: 1 <= G <= 16, d in {64, 128}, T >= 1, B*Hkv <= 32768,
 *  T <= 2^31 - 1.
 */
#ifndef SINKROUTE_H
#define SINKROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SR_OK = 0,
    SR_ERR_INVALID_ARG = 1,  /* null pointer, bad stride/alignment, small workspace */
    SR_ERR_UNSUPPORTED = 2,  /* shape outside the envelope */
    SR_ERR_HIP = 3           /* a HIP call or kernel launch failed */
} sr_status;

typedef enum { SR_KV_BF16 = 0, SR_KV_F32 = 1 } sr_kv_dtype;

/* Which decode kernel runs the active groups. */
typedef enum {
    SR_KERNEL_AUTO = 0,  /* MFMA (it leads at every measured shape) */
    SR_KERNEL_VALU = 1,  /* vector-ALU dot products for QK and PV */
    SR_KERNEL_MFMA = 2   /* matrix cores: bf16 caches, QK (and PV for G > 4) in bf16
                            with fp32 accumulation; fp32 caches, QK and PV in fp32 */
} sr_kernel;

typedef struct {
    int32_t batch;         /* B   >= 1 */
    int32_t num_q_heads;   /* Hq  >= 1, multiple of Hkv */
    int32_t num_kv_heads;  /* Hkv >= 1 */
    int32_t head_dim;      /* d: 64 or 128 */
    int64_t seq_len;       /* T >= 1 */
    int64_t stride_b;      /* cache strides in elements (d is contiguous) */
    int64_t stride_h;
    int64_t stride_t;      /* >= d */
    int32_t kv_dtype;      /* sr_kv_dtype */
    int32_t reserved;      /* must be 0 */
} sr_shape;

/* Launch policy for the decode kernels.  A NULL pointer means all zeros.
 *
 * Work division: an item's cache is cut into chunks of one tile per wave
 * (sr_plan_parts reports the size, 16 to 512 positions), and its chunks are
 * dealt to S lanes round-robin (lane l: chunks l, l + S, l + 2S, ...).  In
 * lanes mode every workgroup takes one lane of one item, so an item's
 * workgroups stream one interleaved window of its cache.  In balanced mode
 * (adaptive policy, when n_active * S leaves workgroups over and the items
 * are long enough) the lanes of all active items are laid end to end and
 * cut into one equal share per workgroup, so a share may span two lanes or
 * two items.  Each workgroup's work on an item is a "part"; the parts of an
 * item are merged in workgroup order. */
typedef struct {
    /* > 0: S = num_splits lanes per item in lanes mode (a lane with no chunk
     *      below T is an empty part).
     *   0: adaptive: the grid is a fixed number of workgroups sized from the
     *      device's CU count; the kernel reads the device-side n_active and
     *      takes S = min(grid / n_active, cap) lanes per item, in balanced
     *      mode when grid / n_active is not a whole number below the cap, so
     *      the GPU stays full at any sink fraction without a host sync.  The
     *      cap (sr_split_cap) weighs the parts' streaming against the merge:
     *      more lanes mean fewer chunks per part, but each started multiple
     *      of the merge's round size (the partials one round trip takes in)
     *      adds a round to the last part's merge.  It is the lane count,
     *      at most the item's chunk count and the grid, that minimises the
     *      estimated chunk and round times measured on MI355X. */
    int32_t num_splits;
    int32_t kernel;        /* sr_kernel */
    int32_t wgs_per_cu;    /* adaptive grid size in workgroups per CU (0 = 1) */
    int32_t waves_per_wg;  /* 4 or 8 wave64s per workgroup (0 = 4); the vector-ALU
                            * kernel runs groups of 9-16 heads with 4 */
} sr_launch;

/* Prefill side (README decode-time steps: the prefill path keeps the key at
 * position 0).  k0[b][g][:] = K[b][g][0][:], v0[b][g][:] = V[b][g][0][:],
 * widened exactly to fp32.  Idempotent. */
sr_status sr_record_sink(const sr_shape* shape, const void* k_cache, const void* v_cache,
                         float* k0, float* v0, void* stream);

/* Routing (README decode-time steps and routing controls; pith.science
 * Figure 10: cos(q, K_BOS) at the KV-group level).
 *   q       fp32 [B][Hq][d], post-RoPE queries.
 *   k0      fp32 [B][Hkv][d] from sr_record_sink.
 *   tau     cosine threshold; a group is a sink iff every one of its G heads
 *           has cos >= tau.  tau > 1 routes nothing (every group active).
 *   scores  out fp32 [B][Hq]: cos(q[b,h], k0[b,h/G]); 0 if either norm is 0.
 *           A NaN or infinite element in q[b,h] or k0 makes the score NaN
 *           (as do squared norms beyond the fp32 range), and a NaN fails the
 *           test at every tau: that head keeps its group active.
 *   mask    out u8 [B][Hkv]: 1 = sink.
 *   work_list out i32 [B*Hkv]: active items ascending, then sinks ascending.
 *   n_active  out i32 [1]: number of active items (stays on the device).
 * B*Hq heads of 3*d multiply-adds each, spread over one workgroup per 16
 * groups (at most 1024 workgroups).  Up to 16 groups that is one launch;
 * above, a second launch on `stream` partitions the groups, with mask as the
 * channel between the two.  Scores and decisions are the same bit for bit in
 * every form. */
sr_status sr_route(const sr_shape* shape, const float* q, const float* k0, float tau,
                   float* scores, uint8_t* mask, int32_t* work_list, int32_t* n_active,
                   void* stream);

/* Decode-step neighbour: rotary embedding of the new token, then the append
 * of its key and value (README decode-time steps: routing compares the
 * RoPE-rotated query with the position-0 key).  Rotary form: element i pairs
 * with element i + d/2 and both turn by the angle pos * inv_freq[i]; angles,
 * sines, cosines and rotations are computed in fp64.
 *   q_new, k_new, v_new: fp32 [B][Hq][d], [B][Hkv][d], [B][Hkv][d], unrotated.
 *   inv_freq: fp32 [d/2] rotary frequencies (any scaling scheme).
 *   pos: position of the new token, 0 <= pos < shape->seq_len, where
 *        shape->seq_len is the caches' capacity.
 *   q_out: fp32 [B][Hq][d], the rotated query (rounded once to fp32).
 *   k_cache[b][g][pos][:] = rotated key, v_cache[b][g][pos][:] = value, each
 *   rounded once to the cache dtype (nearest even); nothing else is written. */
sr_status sr_rope_append(const sr_shape* shape, const float* q_new, const float* k_new,
                         const float* v_new, const float* inv_freq, int64_t pos, float* q_out,
                         void* k_cache, void* v_cache, void* stream);

/* Bytes of scratch the decode calls need for this shape and launch policy:
 * a ticket region of fixed size at the start (one 32-bit ticket for each of
 * the envelope's 32768 items, then the routing kernel's ticket: 131,328
 * bytes with padding), partial results of up to grid + B*Hkv parts (m, l,
 * the position-0 logit and acc, fp32), and, for sr_route_decode on large
 * layers, room for a work list, a count and one flag byte per group.
 * Depends on the current device's CU count in adaptive mode. Returns 0 on an
 * invalid or unsupported shape. */
size_t sr_workspace_bytes(const sr_shape* shape, const sr_launch* launch);

/* Zero a new workspace once (the tickets).  Every decode call leaves the
 * tickets it used back at zero, and the tickets sit at the same offsets for
 * every shape and launch policy, so a workspace is reusable as is by any
 * later call, of any shape, whose sr_workspace_bytes it covers.  Two calls
 * that may run at the same time must not share a workspace. */
sr_status sr_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Routed decode (README decode-time steps; paper Eq. (1)).
 *   work_list, n_active: device outputs of sr_route (the kernels clamp
 *   n_active to [0, B*Hkv] and list entries to [0, B*Hkv), so another list
 *   gives undefined results but no access outside the buffers).  Items at positions
 *   [n_active, B*Hkv) of the list are sinks: their G output rows get v0
 *   (bit-exact) and their caches are never read.  Items before are active:
 *     out[b,h,:] = sum_t softmax_t(sm_scale * <q[b,h], K[b,g,t]>) V[b,g,t,:]
 *   over t = 0..T-1, fp32 accumulation, split over the context and merged in
 *   ascending split order (bitwise reproducible for a given launch policy).
 *   sm_scale <= 0 means 1/sqrt(d); a NaN or infinite one is SR_ERR_INVALID_ARG.
 *   For bf16 caches the MFMA kernel splits each scaled query (and, for
 *   groups of more than 4 heads, each probability) into a sum of two bf16
 *   terms; products with the stored bf16 keys and values are exact and the
 *   results carry ~2^-16 relative error in those operands, far below the
 *   tolerance.  For fp32 caches it multiplies in fp32.
 *   ws: at least sr_workspace_bytes(shape, launch) bytes, initialised once
 *   by sr_workspace_init. */
sr_status sr_decode_attn(const sr_shape* shape, const sr_launch* launch, const float* q,
                         const void* k_cache, const void* v_cache, const float* v0,
                         const int32_t* work_list, const int32_t* n_active, float sm_scale,
                         void* ws, size_t ws_bytes, float* out, void* stream);

/* Routing and decode in one call (sr_route followed by sr_decode_attn, same
 * arguments).  For layers of up to 64 query heads (B*Hq <= 64) it is one
 * launch: every workgroup derives the routing decision itself from q and k0
 * with the arithmetic of sr_route, and workgroup 0 writes the routing
 * outputs.  That saves a launch and the routing kernel per layer-step.
 * Larger layers run the routing kernel and then the decode on `stream`,
 * since scoring hundreds of heads in every workgroup costs more than the
 * extra launch.  Up to 64 KV groups (B*Hkv <= 64) the routing kernel only
 * writes the per-group flags and every decode workgroup partitions them
 * itself; above, the workgroup that finishes scoring last partitions,
 * through a ticket in the workspace.  Either way the decisions, the work list and the output are
 * bit-identical to the two-call form under the same launch policy.  scores /
 * mask / work_list / n_active may each be NULL; the workspace holds the
 * flags, list and count when they are. */
sr_status sr_route_decode(const sr_shape* shape, const sr_launch* launch, const float* q,
                          const void* k_cache, const void* v_cache, const float* k0,
                          const float* v0, float tau, float sm_scale, float* scores,
                          uint8_t* mask, int32_t* work_list, int32_t* n_active, void* ws,
                          size_t ws_bytes, float* out, void* stream);

/* For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture that must not allocate, tight serving loops,
 * harnesses that forbid hipMalloc): sr_route_decode without the ws / ws_bytes
 * arguments.  Its scratch (tickets and split partials) is a device array the
 * library owns, one per GPU, reserved when the library is loaded and held
 * until the process ends; the call itself allocates nothing.  The first call
 * on a device looks the array up and clears its ticket region with a small
 * fill kernel on `stream`; every call leaves the tickets at zero again.
 *   Limit: shapes whose sr_workspace_bytes(shape, launch) exceeds
 *   SR_STATIC_SCRATCH_BYTES are rejected with SR_ERR_UNSUPPORTED before
 *   anything is enqueued.  That size is about (grid + B*Hkv) * GP * (d + 3) * 4
 *   bytes, GP = G rounded up to a power of two: every Llama-3.1-8B or
 *   70B-shaped layer of up to 64 KV groups fits at any adaptive grid of up to
 *   8 workgroups per CU.
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps
 *   the last call's contents.  Calls that may overlap on one device (other
 *   streams, other threads) race and give wrong results; order them.
 * Otherwise the contract, the arguments and the results are sr_route_decode's,
 * bit for bit under the same launch policy. */
#define SR_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
sr_status sr_route_decode_static(const sr_shape* shape, const sr_launch* launch, const float* q,
                                 const void* k_cache, const void* v_cache, const float* k0,
                                 const float* v0, float tau, float sm_scale, float* scores,
                                 uint8_t* mask, int32_t* work_list, int32_t* n_active, float* out,
                                 void* stream);

/* One decode step of a layer in one call: sr_rope_append of the new token
 * at position T - 1 (T = shape->seq_len, the positions attended after the
 * append), then sr_route_decode over positions 0 .. T - 1 (README decode-time
 * steps: rotate the new query, compare it with the position-0 key, route,
 * attend).  Up to 64 query heads it is one launch: every workgroup rotates
 * the queries itself, and the new key and value row of each KV group is
 * written by the one workgroup that reads it in this launch (for a sink
 * group, the one that copies its v0 rows), before it reads.
 *   q_new, k_new, v_new, inv_freq: as sr_rope_append (unrotated, fp32).
 *   q_out: the rotated query [B][Hq][d] (may be NULL up to 64 query heads;
 *   must not overlap q_new or out).
 *   k_cache, v_cache: caches with room for position T - 1 (strides as usual).
 *   k0, v0, tau, sm_scale, scores, mask, work_list, n_active, ws, out: as
 *   sr_route_decode.
 * Bitwise equal to sr_rope_append at pos = T - 1 followed by sr_route_decode
 * with seq_len = T: the same q_out, cache rows, routing outputs and out.
 * Above 64 query heads (B*Hq > 64) it is two launches, like sr_route_decode:
 * the routing kernel's workgroup that scores a KV group first turns that
 * group's queries into q_out and appends its row, then the decode reads
 * q_out, which is therefore required there (NULL: SR_ERR_INVALID_ARG).
 * T >= 2 (position 0 is the recorded sink key).  tau > 1 gives the dense
 * result of the same step. */
sr_status sr_rope_route_decode(const sr_shape* shape, const sr_launch* launch,
                               const float* q_new, const float* k_new, const float* v_new,
                               const float* inv_freq, float* q_out, void* k_cache, void* v_cache,
                               const float* k0, const float* v0, float tau, float sm_scale,
                               float* scores, uint8_t* mask, int32_t* work_list,
                               int32_t* n_active, void* ws, size_t ws_bytes, float* out,
                               void* stream);

/* Dense baseline (README efficiency-benchmark section: the decode latency of
 * the unmodified model, which SinkRouter's speedup is measured against; the
 * paper's Eq. (1) over every group): the decode kernel of sr_decode_attn with
 * routing off (identity work list, every item active).  sr_decode_attn with
 * a work list routed at tau > 1 gives the same bits for the same launch
 * policy.  Arguments, layout, ownership and errors as sr_decode_attn, without
 * v0, work_list and n_active. */
sr_status sr_dense_decode(const sr_shape* shape, const sr_launch* launch, const float* q,
                          const void* k_cache, const void* v_cache, float sm_scale,
                          void* ws, size_t ws_bytes, float* out, void* stream);

/* Dense decode that also reports, per query head, the attention weight of
 * position 0: alpha0[b][h] = softmax weight of the first cached position
 * (Eq. (1) of the paper; the pith.science Figure 10 caption evaluates the
 * cosine routing proxy against sink events defined from this full-attention
 * weight).  alpha0: fp32 [B][Hq], required.  Same contract as
 * sr_dense_decode otherwise; the output is bitwise equal to it. */
sr_status sr_dense_decode_alpha0(const sr_shape* shape, const sr_launch* launch, const float* q,
                                 const void* k_cache, const void* v_cache, float sm_scale, void* ws,
                                 size_t ws_bytes, float* out, float* alpha0, void* stream);

/* Split count.  The pages show the split count only as a launch knob (the
 * README's routing controls give 32 splits as an example at 524288
 * positions).  Here it is not one number per shape: the adaptive policy
 * (sr_launch.num_splits = 0) derives it on the device from n_active, so there
 * is no default-split call; these two calls report what a launch will do.
 *
 * Lanes per active item (S) the decode kernel will use for a given n_active
 * under this policy (what the adaptive mode derives on the device); 0 for an
 * invalid shape or policy. */
int32_t sr_splits_for(const sr_shape* shape, const sr_launch* launch, int32_t n_active);

/* The most lanes per item the policy takes: the adaptive cap above, or the
 * fixed count; 0 for an invalid shape or policy.  The adaptive policy runs in
 * balanced mode exactly when n_active * S < grid and S < this cap. */
int32_t sr_split_cap(const sr_shape* shape, const sr_launch* launch);

/* One workgroup's part of one item, as the decode kernel divides the work. */
typedef struct {
    int32_t item;   /* list position of the item (0 .. n_active - 1) */
    int32_t part;   /* index of this part among the item's parts (workgroup order) */
    int32_t parts;  /* number of parts of the item (1: no merge) */
    int32_t lanes;  /* S, lanes per item */
    int64_t first;  /* the part's range of the item's lane-major chunk sequence */
    int64_t end;    /*   [first, end): position q is chunk l + k * S of lane l */
    int64_t chunk;  /* cache positions per chunk */
} sr_part;

/* Host-side introspection of the work division (no device work): fills
 * parts[0 .. r) with workgroup `wg`'s parts for `n_active` active items and
 * returns r (0 when the workgroup has no cache work; at most 2), or -1 for an
 * invalid shape, policy, n_active (0 .. B*Hkv), wg (0 .. grid - 1) or
 * max_parts < 2.  Lane-major order: lane l of an item holds Q + (l < rem)
 * chunks, Q = C / S and rem = C mod S for C = ceil(T / chunk) chunks, and the
 * lanes follow each other. */
int32_t sr_plan_parts(const sr_shape* shape, const sr_launch* launch, int32_t n_active, int32_t wg,
                      sr_part* parts, int32_t max_parts);

/* Workgroups the decode kernel launches under this policy (0 for an invalid
 * shape or policy). */
int32_t sr_grid_size(const sr_shape* shape, const sr_launch* launch);

const char* sr_status_string(sr_status status);

/* Measurement helper, not part of the decode path: streams `bytes` (rounded
 * down to 16) of device memory with 16-byte loads per lane (the decode
 * kernels' access width) on `grid` workgroups of 256 threads, `unroll` loads
 * in flight per thread (1, 2, 4, 8 or 16), so a benchmark can measure the
 * achievable HBM read bandwidth.  `flags` bit 0 (SR_READ_BLOCKED): each
 * workgroup streams its own contiguous slice instead of the grid walking the
 * buffer together; bit 1 (SR_READ_NONTEMPORAL): loads use the non-temporal
 * cache policy, as the decode kernels' cache loads do; bit 2 (SR_READ_LDS):
 * every load goes straight into the wave's LDS tile (16-byte direct-to-LDS
 * loads, U KiB of LDS per wave) and is read back from there, the shape of a
 * kernel that stages its tiles through LDS.  Other bits are an error.  `sink` (>= grid u32, device) is written only in the practically
 * impossible case that a workgroup's XOR of the data is 0x9e3779b9; it exists
 * so no load can be optimised away. */
#define SR_READ_BLOCKED 1
#define SR_READ_NONTEMPORAL 2
#define SR_READ_LDS 4
sr_status sr_stream_read(const void* buf, size_t bytes, int32_t grid, int32_t unroll,
                         int32_t flags, uint32_t* sink, void* stream);

/* Library version, e.g. 100 for 0.1.0. */
int32_t sr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKROUTE_H */
