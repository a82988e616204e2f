// C ABI of libsinkroute: argument checks, launch sizing and dispatch.
// Declarations and the contract of every call are in include/sinkroute.h.
#include <math.h>

#include <atomic>
#include <mutex>

#include "sr_internal.h"

namespace sr {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

constexpr int32_t kMaxItems = 32768;  // the supported envelope (tested at the maximum)

size_t elem_size(const sr_shape& s) { return s.kv_dtype == SR_KV_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sr_status check_shape(const sr_shape* s) {
    if (!s) return SR_ERR_INVALID_ARG;
    if (s->reserved != 0) return SR_ERR_INVALID_ARG;
    if (s->batch < 1 || s->num_kv_heads < 1 || s->num_q_heads < 1) return SR_ERR_INVALID_ARG;
    if (s->num_q_heads % s->num_kv_heads != 0) return SR_ERR_INVALID_ARG;
    if (s->seq_len < 1) return SR_ERR_INVALID_ARG;
    if (s->kv_dtype != SR_KV_BF16 && s->kv_dtype != SR_KV_F32) return SR_ERR_INVALID_ARG;
    const int32_t G = s->num_q_heads / s->num_kv_heads;
    if (G > 16) return SR_ERR_UNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return SR_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(s->batch) * s->num_kv_heads > kMaxItems) return SR_ERR_UNSUPPORTED;
    if (s->seq_len > INT32_MAX) return SR_ERR_UNSUPPORTED;
    if (s->stride_t < s->head_dim || s->stride_h < 0 || s->stride_b < 0) return SR_ERR_INVALID_ARG;
    const int64_t es = static_cast<int64_t>(elem_size(*s));
    if ((s->stride_t * es) % 16 || (s->stride_h * es) % 16 || (s->stride_b * es) % 16)
        return SR_ERR_INVALID_ARG;
    return SR_OK;
}

sr_status check_caches(const sr_shape& s, const void* k, const void* v) {
    if (!k || !v || !aligned16(k) || !aligned16(v)) return SR_ERR_INVALID_ARG;
    return SR_OK;
}

struct Plan {
    int32_t fixed_splits, grid, split_cap, gp, kernel, waves;
};

sr_status make_plan(const sr_shape& s, const sr_launch* launch, Plan& p) {
    sr_launch l{};
    if (launch) l = *launch;
    if (l.num_splits < 0 || l.wgs_per_cu < 0) return SR_ERR_INVALID_ARG;
    if (l.waves_per_wg != 0 && l.waves_per_wg != 4 && l.waves_per_wg != 8) return SR_ERR_INVALID_ARG;
    p.waves = l.waves_per_wg ? l.waves_per_wg : kDefaultWaves;
    if (l.kernel < SR_KERNEL_AUTO || l.kernel > SR_KERNEL_MFMA) return SR_ERR_INVALID_ARG;
    // Measured on MI355X (interleaved A/B, non-temporal loads, dense decode over
    // ~1 GiB): the matrix-core kernels lead at every group size and head size.
    // bf16 at d = 128: by 0-7 % at G = 1-4, 1.9x at G = 8, 6.6x at G = 16 (PV on
    // the matrix cores from G = 8); bf16 at d = 64 (two tiles per wave step): by
    // 4-7 % at G = 1-4, 2x at G = 8 and 5x at G = 16; fp32: 6.6-6.9 TB/s against
    // 5.9-6.0 at G <= 8 and ~2 at G = 16.  The vector-ALU kernel remains on
    // request.
    p.kernel = l.kernel != SR_KERNEL_AUTO ? l.kernel : SR_KERNEL_MFMA;
    const int64_t n_items = static_cast<int64_t>(s.batch) * s.num_kv_heads;
    p.gp = pad_group(s.num_q_heads / s.num_kv_heads);
    // the vector-ALU kernel's 16-head state only fits one wave per SIMD
    if (p.kernel == SR_KERNEL_VALU && p.gp >= 16) p.waves = 4;
    if (l.num_splits > 0) {
        const int64_t grid = n_items * l.num_splits;
        if (grid > INT32_MAX) return SR_ERR_UNSUPPORTED;
        p.fixed_splits = l.num_splits;
        p.grid = static_cast<int32_t>(grid);
        p.split_cap = l.num_splits;
    } else {
        const int32_t per_cu = l.wgs_per_cu > 0 ? l.wgs_per_cu : kDefaultWgsPerCu;
        int64_t grid = static_cast<int64_t>(per_cu) * cu_count();
        if (grid < n_items) grid = n_items;
        if (grid > INT32_MAX) return SR_ERR_UNSUPPORTED;
        const int32_t kv_bytes = static_cast<int32_t>(elem_size(s));
        const int32_t chunk = chunk_positions(p.kernel, s.head_dim, p.gp, p.waves, kv_bytes);
        p.fixed_splits = 0;
        p.grid = static_cast<int32_t>(grid);
        p.split_cap = adaptive_split_cap(s.seq_len, chunk,
                                         static_cast<int64_t>(chunk) * 2 * s.head_dim * kv_bytes,
                                         merge_round_splits(s.head_dim, p.gp, p.waves), p.grid);
    }
    return SR_OK;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// A workspace (the caller's, or the library's own array for callers that
// cannot allocate) starts with a ticket region of fixed size: one ticket per
// item for the largest layer the envelope allows, then the routing kernel's
// ticket.  The tickets sit at the same offsets whatever the shape and launch,
// and nothing else is ever stored there, so every call finds them at zero
// (zeroed once, and each call leaves the tickets it took back at zero) and a
// workspace serves any later call whose size it covers.  The partials and the
// routing region that follow are written before they are read.
constexpr size_t kTicketBytes = align256((kMaxItems + 1) * sizeof(uint32_t));

struct WsLayout {
    size_t ml, acc, route, total;
};

// Where one decode call keeps its scratch: the per-item tickets and the
// routing kernel's ticket, the partials, and the routing list, count and
// flags of sr_route_decode's two-launch form.
struct Scratch {
    uint32_t* tickets;       // [B*Hkv] of the region's kMaxItems
    uint32_t* route_ticket;  // [1], after the item tickets
    float* part_ml;
    float* part_acc;
    int32_t* route_list;     // [B*Hkv + 1]: list, then n_active
    uint8_t* route_flags;    // [B*Hkv]
};

WsLayout ws_layout(const sr_shape& s, const Plan& p) {
    const size_t n_items = static_cast<size_t>(s.batch) * s.num_kv_heads;
    WsLayout w;
    w.ml = kTicketBytes;
    const size_t parts = static_cast<size_t>(p.grid) + n_items;  // slots w + i, w < grid, i < n
    w.acc = w.ml + align256(parts * 3 * p.gp * sizeof(float));
    // sr_route_decode's two-launch form: work list and n_active [n_items + 1]
    // int32, then one flag byte per item, for callers that do not ask for the
    // list, the count or the mask
    w.route = w.acc + align256(parts * p.gp * s.head_dim * sizeof(float));
    w.total = w.route + align256((n_items + 1) * sizeof(int32_t) + n_items);
    return w;
}

Scratch scratch_at(const sr_shape& s, const WsLayout& w, void* ws) {
    const size_t n_items = static_cast<size_t>(s.batch) * s.num_kv_heads;
    char* base = static_cast<char*>(ws);
    Scratch c;
    c.tickets = reinterpret_cast<uint32_t*>(base);
    c.route_ticket = c.tickets + kMaxItems;
    c.part_ml = reinterpret_cast<float*>(base + w.ml);
    c.part_acc = reinterpret_cast<float*>(base + w.acc);
    c.route_list = reinterpret_cast<int32_t*>(base + w.route);
    c.route_flags = reinterpret_cast<uint8_t*>(c.route_list + n_items + 1);
    return c;
}

// ---------------------------------------------------------------------------
// Library-owned scratch of sr_route_decode_static, for callers that cannot
// allocate.  One array per device (each GPU the library runs on holds its own
// copy until the process ends) with the workspace layout, of
// SR_STATIC_SCRATCH_BYTES: its ticket region is zeroed once at set-up and
// every call leaves it at zero.  Calls that overlap on one device share the
// array and race.
static __device__ __align__(256) unsigned char scratch[SR_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<char*> g_scratch[kMaxDevices];  // device address of `scratch`, per device

// This device's address of `scratch`, set up on its first use: the symbol's
// address is looked up with the device current and the ticket region cleared
// with a fill kernel on `st` (no memset node, so a call under stream capture
// records a plain kernel).
sr_status static_scratch(hipStream_t st, char*& out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SR_ERR_HIP;
    out = g_scratch[dev].load(std::memory_order_acquire);
    if (out) return SR_OK;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    out = g_scratch[dev].load(std::memory_order_acquire);
    if (out) return SR_OK;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SR_ERR_HIP;
    if (launch_zero(ptr, kTicketBytes, st) != hipSuccess) return SR_ERR_HIP;
    out = static_cast<char*>(ptr);
    g_scratch[dev].store(out, std::memory_order_release);
    return SR_OK;
}

struct FusedRoute {
    const float* k0;
    float tau;
    float* scores;
    uint8_t* mask;
    int32_t* work_list;
    int32_t* n_active;
};

struct FusedRope {
    const float* k_new;
    const float* v_new;
    const float* inv_freq;
    float* q_out;
};

bool overlaps(const void* a, const void* b, size_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
}

// ws == nullptr with ws_bytes == kUseStaticScratch: the library's own scratch
// (sr_route_decode_static).
constexpr size_t kUseStaticScratch = ~static_cast<size_t>(0);

sr_status run_decode(const sr_shape* shape, const sr_launch* launch, const float* q,
                     const void* k, const void* v, const float* v0, const int32_t* work_list,
                     const int32_t* n_active, float sm_scale, void* ws, size_t ws_bytes,
                     float* out, void* stream, bool routed, const FusedRoute* fused = nullptr,
                     float* alpha0 = nullptr, const FusedRope* rope = nullptr) {
    const bool use_static = !ws && ws_bytes == kUseStaticScratch;
    sr_status st = check_shape(shape);
    if (st != SR_OK) return st;
    const sr_shape& s = *shape;
    if (rope) {
        // above kMaxFusedHeads the routing kernel rotates the queries into
        // q_out, which the decode launch then reads
        if (static_cast<int64_t>(s.batch) * s.num_q_heads > kMaxFusedHeads && !rope->q_out)
            return SR_ERR_INVALID_ARG;
        if (s.seq_len < 2 || !rope->k_new || !rope->v_new || !rope->inv_freq)
            return SR_ERR_INVALID_ARG;
        const size_t q_bytes =
            static_cast<size_t>(s.batch) * s.num_q_heads * s.head_dim * sizeof(float);
        if (rope->q_out && (overlaps(rope->q_out, q, q_bytes) || overlaps(rope->q_out, out, q_bytes)))
            return SR_ERR_INVALID_ARG;
    }
    if ((st = check_caches(s, k, v)) != SR_OK) return st;
    if (!q || !out || !aligned16(q) || !aligned16(out)) return SR_ERR_INVALID_ARG;
    if (!use_static && (!ws || !aligned16(ws))) return SR_ERR_INVALID_ARG;
    // every workgroup reads q (all of it when it routes) while others write out
    const size_t q_bytes = static_cast<size_t>(s.batch) * s.num_q_heads * s.head_dim * sizeof(float);
    if (overlaps(out, q, q_bytes)) return SR_ERR_INVALID_ARG;
    if (!isfinite(sm_scale)) return SR_ERR_INVALID_ARG;
    if (routed && !v0) return SR_ERR_INVALID_ARG;
    if (routed && !fused && (!work_list || !n_active)) return SR_ERR_INVALID_ARG;
    if (fused && (!fused->k0 || !aligned16(fused->k0) || isnan(fused->tau)))
        return SR_ERR_INVALID_ARG;
    Plan p;
    if ((st = make_plan(s, launch, p)) != SR_OK) return st;
    const WsLayout w = ws_layout(s, p);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    if (use_static) {
        if (w.total > SR_STATIC_SCRATCH_BYTES) return SR_ERR_UNSUPPORTED;
        if ((st = static_scratch(hs, base)) != SR_OK) return st;
    } else if (ws_bytes < w.total) {
        return SR_ERR_INVALID_ARG;
    }
    const Scratch sc = scratch_at(s, w, base);

    DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.v0 = v0;
    a.work_list = work_list;
    a.n_active = n_active;
    a.out = out;
    a.tickets = sc.tickets;
    a.part_ml = sc.part_ml;
    a.part_acc = sc.part_acc;
    a.stride_b = s.stride_b;
    a.stride_h = s.stride_h;
    a.stride_t = s.stride_t;
    a.seq_len = s.seq_len;
    a.batch = s.batch;
    a.num_q_heads = s.num_q_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.group = s.num_q_heads / s.num_kv_heads;
    const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(s.head_dim));
    a.qscale = scale * 1.4426950408889634f;
    a.fixed_splits = p.fixed_splits;
    a.grid = p.grid;
    a.split_cap = p.split_cap;
    a.routed = routed ? 1 : 0;
    a.alpha0_out = alpha0;
    a.kv_f32 = s.kv_dtype == SR_KV_F32 ? 1 : 0;
    if (rope) {
        a.rope = 1;
        a.k_new = rope->k_new;
        a.v_new = rope->v_new;
        a.inv_freq = rope->inv_freq;
        a.q_out = rope->q_out;
    }
    if (fused) {
        a.fused = 1;
        a.k0 = fused->k0;
        a.tau = fused->tau;
        a.scores_out = fused->scores;
        a.mask_out = fused->mask;
        a.list_out = fused->work_list;
        a.n_active_out = fused->n_active;
    }

    if (fused && static_cast<int64_t>(s.batch) * s.num_q_heads > kMaxFusedHeads) {
        // large layer: the routing kernel (spread over the chip), then the decode
        const int32_t n_items = s.batch * s.num_kv_heads;
        uint32_t* ticket = sc.route_ticket;
        int32_t* list = fused->work_list ? fused->work_list : sc.route_list;
        int32_t* n_act = fused->n_active ? fused->n_active : sc.route_list + n_items;
        uint8_t* flags = fused->mask ? fused->mask : sc.route_flags;
        RouteRope rr{};
        if (rope) {
            rr = RouteRope{q, rope->k_new, rope->v_new, rope->inv_freq, rope->q_out,
                           const_cast<void*>(k), const_cast<void*>(v), s.stride_b, s.stride_h,
                           s.stride_t, s.seq_len - 1, s.kv_dtype == SR_KV_F32 ? 1 : 0};
            a.rope = 0;          // done by the routing kernel
            a.q = rope->q_out;   // the decode reads the rotated queries
        }
        if (n_items <= 64) {
            // the routing kernel writes the flags only; every decode workgroup
            // partitions them with one ballot (as when it scores itself) and
            // workgroup 0 writes the list and count
            hipError_t e = launch_route(s, q, fused->k0, fused->tau, fused->scores, flags,
                                        nullptr, nullptr, nullptr, hs, rr);
            if (e != hipSuccess) return SR_ERR_HIP;
            a.flags_in = flags;
            a.mask_out = nullptr;  // the flags are the mask
        } else {
            hipError_t e = launch_route(s, q, fused->k0, fused->tau, fused->scores, flags, list,
                                        n_act, ticket, hs, rr);
            if (e != hipSuccess) return SR_ERR_HIP;
            a.fused = 0;
            a.work_list = list;
            a.n_active = n_act;
        }
    }
    hipError_t e = p.kernel == SR_KERNEL_MFMA ? launch_decode_mfma(s, a, p.gp, p.waves, hs)
                                               : launch_decode_valu(s, a, p.gp, p.waves, hs);
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

}  // namespace
}  // namespace sr

using namespace sr;

extern "C" {

sr_status sr_record_sink(const sr_shape* shape, const void* k_cache, const void* v_cache,
                         float* k0, float* v0, void* stream) {
    sr_status st = check_shape(shape);
    if (st != SR_OK) return st;
    if ((st = check_caches(*shape, k_cache, v_cache)) != SR_OK) return st;
    if (!k0 || !v0) return SR_ERR_INVALID_ARG;
    hipError_t e = launch_record(*shape, k_cache, v_cache, k0, v0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

sr_status sr_route(const sr_shape* shape, const float* q, const float* k0, float tau,
                   float* scores, uint8_t* mask, int32_t* work_list, int32_t* n_active,
                   void* stream) {
    sr_status st = check_shape(shape);
    if (st != SR_OK) return st;
    if (!q || !k0 || !scores || !mask || !work_list || !n_active) return SR_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k0)) return SR_ERR_INVALID_ARG;  // read as float4
    if (isnan(tau)) return SR_ERR_INVALID_ARG;
    hipError_t e = launch_route(*shape, q, k0, tau, scores, mask, work_list, n_active, nullptr,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

sr_status sr_rope_append(const sr_shape* shape, const float* q_new, const float* k_new,
                         const float* v_new, const float* inv_freq, int64_t pos, float* q_out,
                         void* k_cache, void* v_cache, void* stream) {
    sr_status st = check_shape(shape);
    if (st != SR_OK) return st;
    if ((st = check_caches(*shape, k_cache, v_cache)) != SR_OK) return st;
    if (!q_new || !k_new || !v_new || !inv_freq || !q_out) return SR_ERR_INVALID_ARG;
    if (pos < 0 || pos >= shape->seq_len) return SR_ERR_INVALID_ARG;
    hipError_t e = launch_rope_append(*shape, q_new, k_new, v_new, inv_freq, pos, q_out, k_cache,
                                      v_cache, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

size_t sr_workspace_bytes(const sr_shape* shape, const sr_launch* launch) {
    if (check_shape(shape) != SR_OK) return 0;
    Plan p;
    if (make_plan(*shape, launch, p) != SR_OK) return 0;
    return ws_layout(*shape, p).total;
}

sr_status sr_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || !aligned16(ws)) return SR_ERR_INVALID_ARG;
    hipError_t e = launch_zero(ws, ws_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

sr_status sr_decode_attn(const sr_shape* shape, const sr_launch* launch, const float* q,
                         const void* k_cache, const void* v_cache, const float* v0,
                         const int32_t* work_list, const int32_t* n_active, float sm_scale,
                         void* ws, size_t ws_bytes, float* out, void* stream) {
    return run_decode(shape, launch, q, k_cache, v_cache, v0, work_list, n_active, sm_scale, ws,
                      ws_bytes, out, stream, true);
}

sr_status sr_route_decode(const sr_shape* shape, const sr_launch* launch, const float* q,
                          const void* k_cache, const void* v_cache, const float* k0,
                          const float* v0, float tau, float sm_scale, float* scores,
                          uint8_t* mask, int32_t* work_list, int32_t* n_active, void* ws,
                          size_t ws_bytes, float* out, void* stream) {
    const FusedRoute f{k0, tau, scores, mask, work_list, n_active};
    return run_decode(shape, launch, q, k_cache, v_cache, v0, nullptr, nullptr, sm_scale, ws,
                      ws_bytes, out, stream, true, &f);
}

sr_status sr_route_decode_static(const sr_shape* shape, const sr_launch* launch, const float* q,
                                 const void* k_cache, const void* v_cache, const float* k0,
                                 const float* v0, float tau, float sm_scale, float* scores,
                                 uint8_t* mask, int32_t* work_list, int32_t* n_active, float* out,
                                 void* stream) {
    const FusedRoute f{k0, tau, scores, mask, work_list, n_active};
    return run_decode(shape, launch, q, k_cache, v_cache, v0, nullptr, nullptr, sm_scale, nullptr,
                      kUseStaticScratch, out, stream, true, &f);
}

sr_status sr_rope_route_decode(const sr_shape* shape, const sr_launch* launch,
                               const float* q_new, const float* k_new, const float* v_new,
                               const float* inv_freq, float* q_out, void* k_cache, void* v_cache,
                               const float* k0, const float* v0, float tau, float sm_scale,
                               float* scores, uint8_t* mask, int32_t* work_list,
                               int32_t* n_active, void* ws, size_t ws_bytes, float* out,
                               void* stream) {
    const FusedRoute f{k0, tau, scores, mask, work_list, n_active};
    const FusedRope r{k_new, v_new, inv_freq, q_out};
    return run_decode(shape, launch, q_new, k_cache, v_cache, v0, nullptr, nullptr, sm_scale, ws,
                      ws_bytes, out, stream, true, &f, nullptr, &r);
}

sr_status sr_dense_decode(const sr_shape* shape, const sr_launch* launch, const float* q,
                          const void* k_cache, const void* v_cache, float sm_scale, void* ws,
                          size_t ws_bytes, float* out, void* stream) {
    return run_decode(shape, launch, q, k_cache, v_cache, nullptr, nullptr, nullptr, sm_scale, ws,
                      ws_bytes, out, stream, false);
}

sr_status sr_dense_decode_alpha0(const sr_shape* shape, const sr_launch* launch, const float* q,
                                 const void* k_cache, const void* v_cache, float sm_scale, void* ws,
                                 size_t ws_bytes, float* out, float* alpha0, void* stream) {
    if (!alpha0) return SR_ERR_INVALID_ARG;
    return run_decode(shape, launch, q, k_cache, v_cache, nullptr, nullptr, nullptr, sm_scale, ws,
                      ws_bytes, out, stream, false, nullptr, alpha0);
}

int32_t sr_splits_for(const sr_shape* shape, const sr_launch* launch, int32_t n_active) {
    if (check_shape(shape) != SR_OK) return 0;
    Plan p;
    if (make_plan(*shape, launch, p) != SR_OK) return 0;
    return splits_for(p.fixed_splits, p.grid, p.split_cap, n_active);
}

int32_t sr_split_cap(const sr_shape* shape, const sr_launch* launch) {
    if (check_shape(shape) != SR_OK) return 0;
    Plan p;
    if (make_plan(*shape, launch, p) != SR_OK) return 0;
    return p.split_cap;
}

int32_t sr_plan_parts(const sr_shape* shape, const sr_launch* launch, int32_t n_active, int32_t wg,
                      sr_part* parts, int32_t max_parts) {
    if (!parts || max_parts < 2 || check_shape(shape) != SR_OK) return -1;
    Plan p;
    if (make_plan(*shape, launch, p) != SR_OK) return -1;
    const int32_t n_items = shape->batch * shape->num_kv_heads;
    if (n_active < 0 || n_active > n_items || wg < 0 || wg >= p.grid) return -1;
    const int32_t chunk = chunk_positions(p.kernel, shape->head_dim, p.gp, p.waves,
                                          shape->kv_dtype == SR_KV_F32 ? 4 : 2);
    const SplitPlan sp =
        make_split_plan(p.fixed_splits, p.grid, p.split_cap, n_active, shape->seq_len, chunk);
    if (wg >= sp.P) return 0;
    const int64_t p0 = range_begin(sp, wg), p1 = range_begin(sp, wg + 1);
    int32_t i_begin, i_end;
    range_items(sp, wg, i_begin, i_end);
    int32_t r = 0;
    for (int32_t i = i_begin; i < i_end && r < 2; ++i, ++r) {
        int32_t w_lo, n_parts;
        item_parts(sp, i, w_lo, n_parts);
        const int64_t x0 = static_cast<int64_t>(i) * sp.C;
        parts[r].item = i;
        parts[r].part = wg - w_lo;
        parts[r].parts = n_parts;
        parts[r].lanes = sp.S;
        parts[r].first = p0 > x0 ? p0 - x0 : 0;
        parts[r].end = p1 - x0 < sp.C ? p1 - x0 : sp.C;
        parts[r].chunk = chunk;
    }
    return r;
}

int32_t sr_grid_size(const sr_shape* shape, const sr_launch* launch) {
    if (check_shape(shape) != SR_OK) return 0;
    Plan p;
    if (make_plan(*shape, launch, p) != SR_OK) return 0;
    return p.grid;
}

const char* sr_status_string(sr_status status) {
    switch (status) {
        case SR_OK: return "ok";
        case SR_ERR_INVALID_ARG: return "invalid argument";
        case SR_ERR_UNSUPPORTED: return "unsupported shape (use the standard attention path)";
        case SR_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

sr_status sr_stream_read(const void* buf, size_t bytes, int32_t grid, int32_t unroll,
                         int32_t flags, uint32_t* sink, void* stream) {
    if (!buf || !sink || !aligned16(buf) || bytes < 16 || grid < 1) return SR_ERR_INVALID_ARG;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
        return SR_ERR_INVALID_ARG;
    if (flags & ~(SR_READ_BLOCKED | SR_READ_NONTEMPORAL | SR_READ_LDS)) return SR_ERR_INVALID_ARG;
    hipError_t e = launch_stream_read(buf, bytes, grid, unroll, flags, sink,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SR_OK : SR_ERR_HIP;
}

int32_t sr_version(void) { return 100; }

}  // extern "C"
