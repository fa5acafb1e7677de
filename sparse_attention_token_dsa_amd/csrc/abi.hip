// C ABI of the gfx950 indexer library: argument validation, workspace
// planning, kernel sequencing and the optional per-kernel event timing.
// The operations and their sources are described in include/sa_indexer.h.
#include <mutex>
#include <string>
#include <vector>

#include "sa_indexer.h"
#include "sa_common.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(SA_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

// ------------------------------------------------------------ profiling

struct ProfRec {
    int kid;
    hipEvent_t start, stop;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_free_events;
double g_ms[sa::K_COUNT];
long long g_launches[sa::K_COUNT];

hipEvent_t take_event() {
    if (!g_free_events.empty()) {
        hipEvent_t e = g_free_events.back();
        g_free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Move finished records into the totals (synchronises on each stop event).
void drain_records() {
    for (auto& r : g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) == hipSuccess &&
            hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
            g_ms[r.kid] += ms;
            g_launches[r.kid] += 1;
        }
        g_free_events.push_back(r.start);
        g_free_events.push_back(r.stop);
    }
    g_recs.clear();
}

const char* kKernelNames[sa::K_COUNT] = {
    "fill_u32", "scan_dsa", "scan_routed", "block_score", "topk_select", "topk_filter",
    "pool", "pool2", "tail_pool", "misa_router", "gather_rescore", "prefill_fused",
    "quantize_fp8", "scan_dsa_fp8", "block_extrema", "resmisa_router", "head_rows", "tidy",
    "scan_dsa_fp8q", "scan_dsa_pool", "prefill_fused_fp8q"};

// ------------------------------------------------------------ workspace

struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

// ------------------------------------------------------------ validation

int check_shape(const sa_shape* s) {
    if (!s) return fail(SA_EINVAL, "shape is NULL");
    if (s->batch < 1 || s->T < 1 || s->H < 1 || s->L < 1 || s->topk < 1)
        return fail(SA_EINVAL, "batch, T, H, L and topk must be >= 1");
    if (s->d != sa::kD) return fail(SA_EUNSUPPORTED, "d must be 128");
    if (s->H > sa::kMaxH) return fail(SA_EUNSUPPORTED, "H must be <= 64");
    if (s->causal_offset < 0 || (long long)s->causal_offset + s->T > s->L)
        return fail(SA_EINVAL, "need 0 <= causal_offset and causal_offset + T <= L");
    if ((long long)s->batch * s->T > (1LL << 30) || (long long)s->L > (1LL << 30))
        return fail(SA_EUNSUPPORTED, "rows or L too large");
    return SA_OK;
}

// Kernels that index query rows (or sequences) on the grid's y axis: at most
// 65535 of them per call.
constexpr long long kMaxGridY = 65535;

int check_grid_rows(const sa_shape* s) {
    if ((long long)s->batch * s->T > kMaxGridY)
        return fail(SA_EUNSUPPORTED, "batch * T must be <= 65535 per call on this path");
    return SA_OK;
}

int check_grid_batch(const sa_shape* s) {
    if ((long long)s->batch > kMaxGridY) return fail(SA_EUNSUPPORTED, "batch must be <= 65535");
    return SA_OK;
}

int check_ptrs(const void* q, const void* w, const void* k, const void* out_idx) {
    if (!q || !w || !k || !out_idx) return fail(SA_EINVAL, "q, w, keys and out_idx must be non-NULL");
    return SA_OK;
}

// Dense score rows are padded to a multiple of 64 floats (aligned float4
// reads in the top-k filter).
long long score_stride(int L) { return ((long long)L + 63) / 64 * 64; }

// Survivor slots per row of the fused prefill: every legal key when that is
// fewer, else max(6k, 8192).  About k (1 + ln(n / k)) entries survive a
// running threshold over n keys in random order (5.2 k at n = 64 k), so
// typical rows never fill the list; the kernel compacts one that does.  The
// workspace is O(rows * k), not O(rows * n).
long long surv_cap(long long maxn, int k) {
    const long long all = score_stride((int)maxn);
    const long long bounded = std::max<long long>(6LL * k, 8192);
    return std::min(all, (bounded + 63) / 64 * 64);
}

constexpr int kPrefillMinT = 16;

// Rows whose last legal block is cut by the causal bound need a tail rep.
bool any_partial(const sa_shape* s, int block) {
    for (int i = 0; i < s->T; ++i) {
        const long long t = (long long)s->causal_offset + i;
        const long long last = std::min<long long>((t / block + 1) * (long long)block, s->L) - 1;
        if (last > t) return true;
    }
    return false;
}

// ---------------------------------------------------------------- DSA

struct DsaPlan {
    bool prefill;
    float* scores;
    uint32_t* state;
    unsigned long long* cand;
    uint2* surv;
    size_t bytes;
};

DsaPlan plan_dsa(const sa_shape* s, void* ws) {
    DsaPlan p{};
    Carve cv(ws);
    const long long rows = (long long)s->batch * s->T;
    const long long maxn = (long long)s->causal_offset + s->T;
    p.prefill = s->T >= kPrefillMinT;
    if (p.prefill) {
        p.surv = cv.take<uint2>(rows * surv_cap(maxn, s->topk));
    } else {
        p.scores = cv.take<float>(rows * score_stride(s->L));
        p.state = cv.take<uint32_t>(rows * sa::kRowState);
        p.cand = cv.take<unsigned long long>(rows * maxn);
    }
    p.bytes = cv.off + 256;
    return p;
}

// Decode-style path: score rows (+ row state), filter, finish.
// state_zeroed: the caller's previous kernel on the stream already cleared
// the row state.  phases: bit 1 the state clear and the scan, bit 2 the
// top-k from what the scan left in the workspace.
hipError_t run_dense_topk(const uint16_t* q, const float* w, const uint16_t* keys,
                          const sa_shape* s, const int32_t* heads, int hsel, float* scores,
                          uint32_t* state, unsigned long long* cand, int k, int32_t* out_idx,
                          float* out_score, hipStream_t st, const uint8_t* codes = nullptr,
                          const float* kscale = nullptr, bool state_zeroed = false,
                          const int32_t* seq_lens = nullptr, long long total_keys = 0,
                          bool q_fp8 = false, uint16_t* pool_small_out = nullptr,
                          uint16_t* pool_large_out = nullptr, int pool_small = 0,
                          int pool_large = 0, hipEvent_t after_scan = nullptr,
                          const uint16_t* route_reps = nullptr, int route_B = 0,
                          int phases = 3) {
    const long long rows = (long long)s->batch * s->T;
    const int maxn = s->causal_offset + s->T;
    hipError_t e;
    if (phases & 1) {
        if (!state_zeroed) {
            e = sa::launch_fill_u32(state, rows * sa::kRowState, 0u, st);
            if (e != hipSuccess) return e;
        }
        sa::ScanArgs a{};
        a.q = q;
        a.w = w;
        a.keys = keys;
        a.seq_stride = (long long)s->L * sa::kD;
        a.heads = heads;
        a.hsel = hsel;
        a.T = s->T;
        a.H = s->H;
        a.offset = s->causal_offset;
        a.len_div = 1;
        a.len_cap = s->L;
        // Keys per workgroup from the work there is: rows x L, or for ragged
        // batches the caller's total of the sequence lengths when given.
        const long long work = total_keys > 0 ? total_keys : rows * (long long)s->L;
        const int wrk = (int)std::min<long long>(work, 1LL << 30);
        a.chunk = codes ? sa::scan8_chunk(1, wrk) : sa::scan_chunk(4, 1, wrk);
        a.scores = scores;
        a.score_stride = score_stride(s->L);
        a.state = state;
        a.k = k;
        a.codes = codes;
        a.kscale = kscale;
        a.seq_lens = seq_lens;
        a.q_fp8 = q_fp8 ? 1 : 0;
        if (route_reps) {
            // the scan routes each row itself and writes the heads to `heads`
            a.route_reps = route_reps;
            a.route_B = route_B;
            a.route_nblk = (s->L + route_B - 1) / route_B;
            a.route_seq_stride = (long long)a.route_nblk * 2 * sa::kD;
            a.route_heads_out = const_cast<int32_t*>(heads);
        }
        const int nht = ((heads ? hsel : s->H) + 15) / 16;
        if (pool_small_out) {
            // chunks of whole large blocks (pool_large divides kScanPoolChunk)
            const int c = (a.chunk + pool_large - 1) / pool_large * pool_large;
            a.chunk = std::min(c, sa::kScanPoolChunk);
            a.pool_out_small = pool_small_out;
            a.pool_out_large = pool_large_out;
            a.pool_small = pool_small;
            a.pool_large = pool_large;
            a.pool_shift = 0;
            while ((64 << a.pool_shift) < pool_small) ++a.pool_shift;
            e = sa::launch_scan_pooled(a, (int)rows, nht, st);
        } else {
            e = codes ? sa::launch_scan8(a, (int)rows, nht, st)
                      : sa::launch_scan(a, (int)rows, nht, 4, heads != nullptr, st);
        }
        if (e != hipSuccess) return e;
        if (after_scan) {
            e = hipEventRecord(after_scan, st);
            if (e != hipSuccess) return e;
        }
    }
    if (!(phases & 2)) return hipSuccess;
    sa::TopkArgs t{};
    t.dense = scores;
    t.dense_stride = score_stride(s->L);
    t.T = s->T;
    t.offset = s->causal_offset;
    t.len_div = 1;
    t.len_cap = s->L;
    t.state = state;
    t.k = k;
    t.out_idx = out_idx;
    t.out_score = out_score;
    t.out_stride = k;
    t.cand_cap = maxn;
    t.seq_lens = seq_lens;
    return sa::launch_topk_dense_filtered(t, (int)rows, maxn, cand, st);
}

hipError_t run_list_topk(const float* ls, const int32_t* li, long long stride,
                         const int32_t* counts, int cap, int rows, int k, int32_t* out_idx,
                         float* out_score, hipStream_t st) {
    sa::TopkArgs t{};
    t.list_score = ls;
    t.list_idx = li;
    t.list_stride = stride;
    t.list_count = counts;
    t.list_cap = cap;
    t.k = k;
    t.out_idx = out_idx;
    t.out_score = out_score;
    t.out_stride = k;
    return sa::launch_topk(t, rows, st);
}

// ---------------------------------------------------------------- MISA

struct MisaPlan {
    bool prefill;
    uint16_t* pooled;
    uint16_t* tail;
    uint8_t* flag;
    int32_t* heads;
    float* scores;
    uint32_t* state;
    unsigned long long* cand;
    uint16_t* qp;
    float* wp;
    uint2* surv;
    int32_t* pool_idx;
    float* list_score;
    int32_t* list_idx;
    size_t bytes;
};

// Decode-style rows (T < 16) score the routed heads with the dense scan into
// O(L) score rows; prefill rows (T >= 16) take the fused prefill on the
// routed heads' q rows (written by the router), so no rows x L scores exist.
MisaPlan plan_misa(const sa_shape* s, int B, int h, int kp, bool pooled_given, bool partial,
                   void* ws) {
    MisaPlan p{};
    Carve cv(ws);
    const long long rows = (long long)s->batch * s->T;
    const long long maxn = (long long)s->causal_offset + s->T;
    const long long nblk = (s->L + B - 1) / B;
    p.prefill = s->T >= kPrefillMinT;
    if (!pooled_given) p.pooled = cv.take<uint16_t>(s->batch * nblk * 2 * sa::kD);
    if (partial) {
        p.tail = cv.take<uint16_t>(rows * 2 * sa::kD);
        p.flag = cv.take<uint8_t>(rows);
    }
    p.heads = cv.take<int32_t>(rows * h);
    if (p.prefill) {
        p.qp = cv.take<uint16_t>(rows * h * sa::kD);
        p.wp = cv.take<float>(rows * h);
        p.surv = cv.take<uint2>(rows * surv_cap(maxn, kp ? kp : s->topk));
    } else {
        p.scores = cv.take<float>(rows * score_stride(s->L));
        p.state = cv.take<uint32_t>(rows * sa::kRowState);
        p.cand = cv.take<unsigned long long>(rows * maxn);
    }
    if (kp > 0) {
        p.pool_idx = cv.take<int32_t>(rows * kp);
        p.list_score = cv.take<float>(rows * kp);
        p.list_idx = cv.take<int32_t>(rows * kp);
    }
    p.bytes = cv.off + 256;
    return p;
}

int check_misa(const sa_shape* s, int B, int h, int kp) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (B < 1) return fail(SA_EINVAL, "block_B must be >= 1");
    if (h < 1 || h > s->H) return fail(SA_EINVAL, "need 1 <= h <= H");
    if (kp != 0 && kp < s->topk) return fail(SA_EINVAL, "k_prime must be 0 or >= topk");
    return check_grid_rows(s);
}

// ---------------------------------------------------------------- HISA

struct HisaPlan {
    uint16_t* reps;
    uint16_t* tail;
    uint8_t* flag;
    float* bscores;
    int32_t* blocks;
    float* list_score;
    int32_t* list_idx;
    size_t bytes;
};

HisaPlan plan_hisa(const sa_shape* s, int b, int r, bool reps_given, bool partial, void* ws) {
    HisaPlan p{};
    Carve cv(ws);
    const long long rows = (long long)s->batch * s->T;
    const long long nblk = (s->L + b - 1) / b;
    if (!reps_given) p.reps = cv.take<uint16_t>(s->batch * nblk * 2 * sa::kD);
    if (partial) {
        p.tail = cv.take<uint16_t>(rows * 2 * sa::kD);
        p.flag = cv.take<uint8_t>(rows);
    }
    p.bscores = cv.take<float>(rows * nblk);
    p.blocks = cv.take<int32_t>(rows * r);
    p.list_score = cv.take<float>(rows * (long long)r * b);
    p.list_idx = cv.take<int32_t>(rows * (long long)r * b);
    p.bytes = cv.off + 256;
    return p;
}

int check_hisa(const sa_shape* s, int b, int r) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (b < 1 || r < 1) return fail(SA_EINVAL, "block_b and r must be >= 1");
    if ((long long)r * b < s->topk) return fail(SA_EINVAL, "need r * block_b >= topk");
    if ((long long)r * b > (1LL << 30)) return fail(SA_EUNSUPPORTED, "r * block_b too large");
    return check_grid_rows(s);
}

}  // namespace

// ------------------------------------------------------------- profiling

namespace sa {

// The open record of this host thread: its index in g_recs, or -1.
static thread_local int t_open = -1;
static thread_local bool t_taken = false;

void prof_reset_thread() {
    t_open = -1;
    t_taken = false;
}

void prof_begin(int kid, hipStream_t s) {
    (void)s;
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) return;
    g_recs.push_back(ProfRec{kid, a, b});
    t_open = (int)g_recs.size() - 1;
    t_taken = false;
}

bool prof_pending(hipEvent_t* start, hipEvent_t* stop) {
    if (t_open < 0 || t_taken) return false;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (t_open < 0 || t_open >= (int)g_recs.size()) return false;
    *start = g_recs[t_open].start;
    *stop = g_recs[t_open].stop;
    t_taken = true;
    return true;
}

void prof_end(int kid, hipStream_t s) {
    (void)s;
    if (t_open < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (t_open < (int)g_recs.size() && g_recs[t_open].kid == kid && !t_taken) {
        // no kernel was launched: drop the record
        g_free_events.push_back(g_recs[t_open].start);
        g_free_events.push_back(g_recs[t_open].stop);
        g_recs.erase(g_recs.begin() + t_open);
    }
    t_open = -1;
    t_taken = false;
}

}  // namespace sa

extern "C" {

const char* sa_last_error(void) { return g_err.c_str(); }

int sa_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) {
        drain_records();
        for (int i = 0; i < sa::K_COUNT; ++i) {
            g_ms[i] = 0.0;
            g_launches[i] = 0;
        }
    }
    g_prof_on = on != 0;
    sa::prof_reset_thread();
    return SA_OK;
}

int sa_profile_read(int32_t id, double* total_ms, int64_t* launches) {
    if (id < 0 || id >= sa::K_COUNT || !total_ms || !launches)
        return fail(SA_EINVAL, "bad kernel id or NULL output");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    drain_records();
    *total_ms = g_ms[id];
    *launches = g_launches[id];
    return SA_OK;
}

int32_t sa_kernel_count(void) { return sa::K_COUNT; }

const char* sa_kernel_name(int32_t id) {
    if (id < 0 || id >= sa::K_COUNT) return "";
    return kKernelNames[id];
}

// ------------------------------------------------------------------ DSA

static int check_dsa(const sa_shape* s) {
    int rc = check_shape(s);
    if (rc) return rc;
    return s->T >= kPrefillMinT ? check_grid_batch(s) : check_grid_rows(s);
}

// Fused prefill rows (T >= 16) of a DSA call; seq_lens for ragged batches.
static hipError_t run_prefill(const uint16_t* q, const float* w, const uint16_t* keys,
                              const sa_shape* s, const DsaPlan& p, int32_t* out_idx,
                              float* out_score, hipStream_t st, const int32_t* seq_lens) {
    sa::PrefillArgs a{};
    a.q = q;
    a.w = w;
    a.keys = keys;
    a.T = s->T;
    a.H = s->H;
    a.L = s->L;
    a.offset = s->causal_offset;
    a.k = s->topk;
    a.surv = p.surv;
    a.cap = surv_cap((long long)s->causal_offset + s->T, s->topk);
    a.out_idx = out_idx;
    a.out_score = out_score;
    a.out_stride = s->topk;
    a.seq_lens = seq_lens;
    return sa::launch_prefill(a, s->batch * s->T, st);
}

int indexer_score_topk_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_dsa(s);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

int indexer_score_topk(const uint16_t* q, const float* w, const uint16_t* keys,
                       const sa_shape* s, int32_t* out_idx, float* out_score, void* ws,
                       size_t ws_bytes, void* stream) {
    int rc = check_dsa(s);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    const size_t need = plan_dsa(s, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    DsaPlan p = plan_dsa(s, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (p.prefill) {
        e = run_prefill(q, w, keys, s, p, out_idx, out_score, st, nullptr);
        if (e != hipSuccess) return hip_fail(e, "prefill");
    } else {
        e = run_dense_topk(q, w, keys, s, nullptr, 0, p.scores, p.state, p.cand, s->topk,
                           out_idx, out_score, st);
        if (e != hipSuccess) return hip_fail(e, "decode scan");
    }
    return SA_OK;
}

// ------------------------------------------------- allocation-free DSA

}  // extern "C"

namespace {

// The scratch of indexer_score_topk_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes its name
// to a kernel (on the host the name is only a stand-in): the device address
// of each GPU's copy comes from hipGetSymbolAddress with that device current.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// This GPU's scratch address, looked up once per device.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SA_EUNSUPPORTED, "device ordinal >= 64");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(SA_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SA_OK;
}

}  // namespace

extern "C" {

int indexer_score_topk_noalloc(const uint16_t* q, const float* w, const uint16_t* keys,
                               const sa_shape* s, int32_t* out_idx, float* out_score,
                               void* stream) {
    int rc = check_dsa(s);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    const size_t need = plan_dsa(s, nullptr).bytes;
    if (need > (size_t)SA_NOALLOC_SCRATCH_BYTES)
        return fail(SA_EWORKSPACE, "this shape needs " + std::to_string(need) +
                                       " bytes of scratch; the static scratch holds " +
                                       std::to_string((size_t)SA_NOALLOC_SCRATCH_BYTES));
    void* base = nullptr;
    rc = scratch_address(&base);
    if (rc) return rc;
    // Same plan and kernels as indexer_score_topk on a workspace at the
    // scratch's (256-byte aligned) address; the decode path clears its row
    // state with a fill kernel before the scan.
    DsaPlan p = plan_dsa(s, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (p.prefill) {
        e = run_prefill(q, w, keys, s, p, out_idx, out_score, st, nullptr);
        if (e != hipSuccess) return hip_fail(e, "prefill");
    } else {
        e = run_dense_topk(q, w, keys, s, nullptr, 0, p.scores, p.state, p.cand, s->topk,
                           out_idx, out_score, st);
        if (e != hipSuccess) return hip_fail(e, "decode scan");
    }
    return SA_OK;
}

// ------------------------------------------------- DSA + block pooling

static int check_pooled(const sa_shape* s, int small, int large) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->T != 1 || s->causal_offset != s->L - 1)
        return fail(SA_EUNSUPPORTED, "pooled DSA: decode rows only (T = 1, causal_offset = L - 1)");
    if (small < 128 || (small & (small - 1)) != 0 || large < small || large % small != 0)
        return fail(SA_EINVAL, "pooled DSA: need small a power of two >= 128 and large a "
                               "multiple of small");
    if (large > sa::kScanPoolChunk || sa::kScanPoolChunk % large != 0)
        return fail(SA_EUNSUPPORTED, "pooled DSA: large must divide 2048");
    return check_grid_rows(s);
}

int indexer_score_topk_pooled_ws(const sa_shape* s, int32_t small, int32_t large,
                                 size_t* ws_bytes) {
    int rc = check_pooled(s, small, large);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

static int pooled_phases(const uint16_t* q, const float* w, const uint16_t* keys,
                         const sa_shape* s, int32_t small, int32_t large, uint16_t* out_small,
                         uint16_t* out_large, int32_t* out_idx, float* out_score, void* ws,
                         size_t ws_bytes, void* pools_ready, int32_t phases, void* stream) {
    if (phases < 1 || phases > 3) return fail(SA_EINVAL, "phases must be 1, 2 or 3");
    int rc = check_pooled(s, small, large);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    if (!out_small || !out_large) return fail(SA_EINVAL, "out_small and out_large must be non-NULL");
    const size_t need = plan_dsa(s, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    DsaPlan p = plan_dsa(s, base);
    hipError_t e = run_dense_topk(q, w, keys, s, nullptr, 0, p.scores, p.state, p.cand, s->topk,
                                  out_idx, out_score, static_cast<hipStream_t>(stream), nullptr,
                                  nullptr, false, nullptr, 0, false, out_small, out_large, small,
                                  large, static_cast<hipEvent_t>(pools_ready), nullptr, 0, phases);
    if (e != hipSuccess) return hip_fail(e, "pooled decode scan");
    return SA_OK;
}

int indexer_score_topk_pooled(const uint16_t* q, const float* w, const uint16_t* keys,
                              const sa_shape* s, int32_t small, int32_t large,
                              uint16_t* out_small, uint16_t* out_large, int32_t* out_idx,
                              float* out_score, void* ws, size_t ws_bytes, void* pools_ready,
                              void* stream) {
    return pooled_phases(q, w, keys, s, small, large, out_small, out_large, out_idx, out_score,
                         ws, ws_bytes, pools_ready, 3, stream);
}

int indexer_score_topk_pooled_phase(const uint16_t* q, const float* w, const uint16_t* keys,
                                    const sa_shape* s, int32_t small, int32_t large,
                                    uint16_t* out_small, uint16_t* out_large, int32_t* out_idx,
                                    float* out_score, void* ws, size_t ws_bytes, int32_t phases,
                                    void* stream) {
    return pooled_phases(q, w, keys, s, small, large, out_small, out_large, out_idx, out_score,
                         ws, ws_bytes, nullptr, phases, stream);
}

// ------------------------------------------------------------ tidy-up

int sa_tidy_indices(const int32_t* idx, int32_t rows, int32_t T, int32_t k,
                    const int32_t* block_table, int32_t pages_per_seq, int32_t page_size,
                    int32_t max_slots, int32_t* out_slots, int32_t* out_stats, void* stream) {
    if (!idx || !out_slots) return fail(SA_EINVAL, "idx and out_slots must be non-NULL");
    if (rows < 1 || T < 1 || rows % T != 0) return fail(SA_EINVAL, "need rows >= 1, T >= 1, T | rows");
    if (k < 1) return fail(SA_EINVAL, "k must be >= 1");
    if (max_slots < 0) return fail(SA_EINVAL, "max_slots must be >= 0");
    const bool bitmap = max_slots > 0 && max_slots <= sa::kTidyBitmapMax;
    if (!bitmap && k > sa::kTidyMax)
        return fail(SA_EUNSUPPORTED, "k > 4096 needs a slot bound max_slots <= 2^18");
    if (page_size < 1) return fail(SA_EINVAL, "page_size must be >= 1");
    if (block_table && pages_per_seq < 1) return fail(SA_EINVAL, "pages_per_seq must be >= 1");
    sa::TidyArgs a{};
    a.idx = idx;
    a.k = k;
    a.T = T;
    int n2 = 256;
    while (n2 < k) n2 <<= 1;
    a.n2 = n2;
    a.table = block_table;
    a.pages_per_seq = block_table ? pages_per_seq : 0;
    a.page = page_size;
    a.max_slots = max_slots;
    a.out_slots = out_slots;
    a.out_stats = out_stats;
    hipError_t e = sa::launch_tidy(a, rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "tidy");
    return SA_OK;
}

// ----------------------------------------------------------- ragged rows

static int check_ragged(const sa_shape* s) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->causal_offset != s->L - s->T)
        return fail(SA_EINVAL, "ragged batches: causal_offset must be L - T (the capacity)");
    return s->T >= kPrefillMinT ? check_grid_batch(s) : check_grid_rows(s);
}

int indexer_score_topk_ragged_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_ragged(s);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

int indexer_score_topk_ragged(const uint16_t* q, const float* w, const uint16_t* keys,
                              const int32_t* seq_lens, int64_t total_len, const sa_shape* s,
                              int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                              void* stream) {
    int rc = check_ragged(s);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    if (!seq_lens) return fail(SA_EINVAL, "seq_lens is NULL");
    if (total_len < 0) return fail(SA_EINVAL, "total_len must be >= 0");
    const size_t need = plan_dsa(s, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    DsaPlan p = plan_dsa(s, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.prefill) {
        hipError_t e = run_prefill(q, w, keys, s, p, out_idx, out_score, st, seq_lens);
        if (e != hipSuccess) return hip_fail(e, "ragged prefill");
        return SA_OK;
    }
    hipError_t e = run_dense_topk(q, w, keys, s, nullptr, 0, p.scores, p.state, p.cand,
                                  s->topk, out_idx, out_score, st, nullptr, nullptr, false,
                                  seq_lens, total_len);
    if (e != hipSuccess) return hip_fail(e, "ragged decode scan");
    return SA_OK;
}

// ------------------------------------------------------------- FP8 keys

int sa_quantize_keys_fp8(const uint16_t* keys, int32_t batch, int32_t L, int32_t d,
                         uint8_t* codes, float* scales, void* stream) {
    if (!keys || !codes || !scales) return fail(SA_EINVAL, "keys, codes and scales must be non-NULL");
    if (batch < 1 || L < 1) return fail(SA_EINVAL, "batch and L must be >= 1");
    if (d != sa::kD) return fail(SA_EUNSUPPORTED, "d must be 128");
    hipError_t e = sa::launch_quantize_fp8(keys, (long long)batch * L, codes, scales,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "quantize fp8");
    return SA_OK;
}

// FP8 keys: decode-style rows (T < 16) with q in bf16 or E4M3; prefill rows
// (T >= 16) with q in E4M3 only (the fused prefill on the fp8 MFMA).
static int check_fp8_shape(const sa_shape* s, bool prefill_ok = false) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (s->T >= kPrefillMinT) {
        if (!prefill_ok)
            return fail(SA_EUNSUPPORTED,
                        "FP8 keys with a bf16 query: decode-style rows only (T < 16); "
                        "prefill rows take the E4M3 query (indexer_score_topk_fp8q)");
        return check_grid_batch(s);
    }
    return check_grid_rows(s);
}

// Fused prefill rows on the FP8 cache, the query quantized in the kernel.
static hipError_t run_prefill_fp8(const uint16_t* q, const float* w, const uint8_t* codes,
                                  const float* scales, const sa_shape* s, const DsaPlan& p,
                                  int32_t* out_idx, float* out_score, hipStream_t st,
                                  const int32_t* seq_lens) {
    sa::PrefillArgs a{};
    a.q = q;
    a.w = w;
    a.codes = codes;
    a.kscale = scales;
    a.T = s->T;
    a.H = s->H;
    a.L = s->L;
    a.offset = s->causal_offset;
    a.k = s->topk;
    a.surv = p.surv;
    a.cap = surv_cap((long long)s->causal_offset + s->T, s->topk);
    a.out_idx = out_idx;
    a.out_score = out_score;
    a.out_stride = s->topk;
    a.seq_lens = seq_lens;
    return sa::launch_prefill(a, s->batch * s->T, st);
}

int indexer_score_topk_fp8_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_fp8_shape(s);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

static int run_fp8(const uint16_t* q, const float* w, const uint8_t* codes, const float* scales,
                   const sa_shape* s, int32_t* out_idx, float* out_score, void* ws,
                   size_t ws_bytes, void* stream, bool q_fp8) {
    int rc = check_fp8_shape(s, q_fp8);
    if (rc) return rc;
    if (!q || !w || !codes || !scales || !out_idx)
        return fail(SA_EINVAL, "q, w, codes, scales and out_idx must be non-NULL");
    const size_t need = plan_dsa(s, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    DsaPlan p = plan_dsa(s, base);
    if (p.prefill) {
        hipError_t e = run_prefill_fp8(q, w, codes, scales, s, p, out_idx, out_score,
                                       static_cast<hipStream_t>(stream), nullptr);
        if (e != hipSuccess) return hip_fail(e, "fp8 prefill");
        return SA_OK;
    }
    hipError_t e = run_dense_topk(q, w, nullptr, s, nullptr, 0, p.scores, p.state, p.cand,
                                  s->topk, out_idx, out_score, static_cast<hipStream_t>(stream),
                                  codes, scales, false, nullptr, 0, q_fp8);
    if (e != hipSuccess) return hip_fail(e, "fp8 decode scan");
    return SA_OK;
}

int indexer_score_topk_fp8(const uint16_t* q, const float* w, const uint8_t* codes,
                           const float* scales, const sa_shape* s, int32_t* out_idx,
                           float* out_score, void* ws, size_t ws_bytes, void* stream) {
    return run_fp8(q, w, codes, scales, s, out_idx, out_score, ws, ws_bytes, stream, false);
}

int indexer_score_topk_fp8_ragged_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_fp8_shape(s, true);
    if (rc) return rc;
    if (s->causal_offset != s->L - s->T)
        return fail(SA_EINVAL, "ragged batches: causal_offset must be L - T (the capacity)");
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

int indexer_score_topk_fp8_ragged(const uint16_t* q, const float* w, const uint8_t* codes,
                                  const float* scales, const int32_t* seq_lens, int64_t total_len,
                                  int32_t q_fp8, const sa_shape* s, int32_t* out_idx,
                                  float* out_score, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    int rc = indexer_score_topk_fp8_ragged_ws(s, &need);
    if (rc) return rc;
    if (!q || !w || !codes || !scales || !seq_lens || !out_idx)
        return fail(SA_EINVAL, "q, w, codes, scales, seq_lens and out_idx must be non-NULL");
    if (total_len < 0) return fail(SA_EINVAL, "total_len must be >= 0");
    if (s->T >= kPrefillMinT && !q_fp8)
        return fail(SA_EUNSUPPORTED,
                    "FP8 keys with a bf16 query: decode-style rows only (T < 16); prefill "
                    "rows take q_fp8 = 1");
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    DsaPlan p = plan_dsa(s, base);
    hipError_t e;
    if (p.prefill) {
        e = run_prefill_fp8(q, w, codes, scales, s, p, out_idx, out_score,
                            static_cast<hipStream_t>(stream), seq_lens);
        if (e != hipSuccess) return hip_fail(e, "ragged fp8 prefill");
        return SA_OK;
    }
    e = run_dense_topk(q, w, nullptr, s, nullptr, 0, p.scores, p.state, p.cand,
                       s->topk, out_idx, out_score, static_cast<hipStream_t>(stream),
                       codes, scales, false, seq_lens, total_len, q_fp8 != 0);
    if (e != hipSuccess) return hip_fail(e, "ragged fp8 decode scan");
    return SA_OK;
}

int indexer_score_topk_fp8q_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_fp8_shape(s, true);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_dsa(s, nullptr).bytes;
    return SA_OK;
}

int indexer_score_topk_fp8q(const uint16_t* q, const float* w, const uint8_t* codes,
                            const float* scales, const sa_shape* s, int32_t* out_idx,
                            float* out_score, void* ws, size_t ws_bytes, void* stream) {
    return run_fp8(q, w, codes, scales, s, out_idx, out_score, ws, ws_bytes, stream, true);
}

// ------------------------------------------------------- LISA / ResMiSA

// Head rows per query row: the four linear heads (g' hi/lo, both signs) plus
// the r routed heads; with r == H, g' is zero and only the H heads remain.
static int resmisa_heads(int H, int r) { return r == H ? H : 4 + r; }

// Router workgroups per row: 64 blocks each over the widest row's legal blocks.
static int resmisa_chunks(const sa_shape* s, int block) {
    const long long maxnb = ((long long)s->causal_offset + s->T - 1) / block + 1;
    return (int)((maxnb + 63) / 64);
}

struct ResPlan {
    uint16_t* qp;
    float* wp;
    float* part;
    uint16_t* ext;
    uint16_t* tail;
    uint8_t* flag;
    DsaPlan dsa;
    size_t bytes;
};

static ResPlan plan_resmisa(const sa_shape* s, int block, int r, bool ext_given, bool partial,
                            void* ws) {
    ResPlan p{};
    Carve cv(ws);
    const long long rows = (long long)s->batch * s->T;
    const int Hp = resmisa_heads(s->H, r);
    p.qp = cv.take<uint16_t>(rows * Hp * sa::kD);
    p.wp = cv.take<float>(rows * Hp);
    if (r > 0) {
        const long long nblk = ((long long)s->L + block - 1) / block;
        p.part = cv.take<float>(rows * resmisa_chunks(s, block) * s->H);
        if (!ext_given) p.ext = cv.take<uint16_t>((long long)s->batch * nblk * 2 * sa::kD);
        if (partial) {
            p.tail = cv.take<uint16_t>(rows * 2 * sa::kD);
            p.flag = cv.take<uint8_t>(rows);
        }
    }
    const size_t off = (cv.off + 255) & ~size_t(255);
    sa_shape s2 = *s;
    s2.H = Hp;
    p.dsa = plan_dsa(&s2, ws ? static_cast<char*>(ws) + off : nullptr);
    p.bytes = off + p.dsa.bytes;
    return p;
}

static int check_resmisa(const sa_shape* s, int block, int r) {
    int rc = check_shape(s);
    if (rc) return rc;
    if (r < 0 || r > s->H) return fail(SA_EINVAL, "need 0 <= r <= H");
    if (r > 0 && block < 1) return fail(SA_EINVAL, "block must be >= 1");
    if (resmisa_heads(s->H, r) > sa::kMaxH)
        return fail(SA_EUNSUPPORTED, "4 + r head rows must fit in 64 (r <= 60, or r == H)");
    // the router and the decode scan put rows on the grid's y axis; the fused
    // prefill puts sequences there
    return (r > 0 || s->T < kPrefillMinT) ? check_grid_rows(s) : check_grid_batch(s);
}

// LISA (r = 0) and ResMiSA: head rows, then the DSA score path on them.
static int run_resmisa(const uint16_t* q, const float* w, const uint16_t* keys,
                       const sa_shape* s, int block, int r, const uint16_t* extrema,
                       int32_t* out_heads, int32_t* out_idx, float* out_score, void* ws,
                       size_t ws_bytes, void* stream) {
    const bool partial = r > 0 && any_partial(s, block);
    const size_t need = plan_resmisa(s, block, r, extrema != nullptr, partial, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    ResPlan p = plan_resmisa(s, block, r, extrema != nullptr, partial, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int rows = s->batch * s->T;
    const int Hp = resmisa_heads(s->H, r);
    sa::ResmisaArgs a{};
    a.q = q;
    a.w = w;
    a.T = s->T;
    a.H = s->H;
    a.offset = s->causal_offset;
    a.block = block;
    a.nblk = r > 0 ? (s->L + block - 1) / block : 0;
    a.r = r;
    a.Hp = Hp;
    a.part = p.part;
    a.nchunk = r > 0 ? resmisa_chunks(s, block) : 0;
    a.heads_out = out_heads;
    a.qp = p.qp;
    a.wp = p.wp;
    a.zero_state = p.dsa.prefill ? nullptr : p.dsa.state;
    hipError_t e;
    if (r > 0) {
        if (!extrema) {
            e = sa::launch_extrema(keys, s->batch, s->L, block, p.ext, st);
            if (e != hipSuccess) return hip_fail(e, "block extrema");
        }
        a.ext = extrema ? extrema : p.ext;
        if (partial) {
            e = sa::launch_extrema_tail(keys, (long long)s->L * sa::kD, s->T, s->causal_offset,
                                        s->L, block, rows, p.tail, p.flag, st);
            if (e != hipSuccess) return hip_fail(e, "cut-block extrema");
            a.tail = p.tail;
            a.tail_flag = p.flag;
        }
        e = sa::launch_resmisa_router(a, rows, st);
        if (e != hipSuccess) return hip_fail(e, "residual routing");
    }
    e = sa::launch_head_rows(a, rows, st);
    if (e != hipSuccess) return hip_fail(e, "head rows");
    sa_shape s2 = *s;
    s2.H = Hp;
    if (p.dsa.prefill) {
        sa::PrefillArgs pa{};
        pa.q = p.qp;
        pa.w = p.wp;
        pa.keys = keys;
        pa.T = s->T;
        pa.H = Hp;
        pa.L = s->L;
        pa.offset = s->causal_offset;
        pa.k = s->topk;
        pa.surv = p.dsa.surv;
        pa.cap = surv_cap((long long)s->causal_offset + s->T, s->topk);
        pa.out_idx = out_idx;
        pa.out_score = out_score;
        pa.out_stride = s->topk;
        e = sa::launch_prefill(pa, rows, st);
        if (e != hipSuccess) return hip_fail(e, "prefill");
    } else {
        e = run_dense_topk(p.qp, p.wp, keys, &s2, nullptr, 0, p.dsa.scores, p.dsa.state,
                           p.dsa.cand, s->topk, out_idx, out_score, st, nullptr, nullptr,
                           /*state_zeroed=*/true);
        if (e != hipSuccess) return hip_fail(e, "decode scan");
    }
    return SA_OK;
}

int lisa_score_topk_ws(const sa_shape* s, size_t* ws_bytes) {
    int rc = check_resmisa(s, 1, 0);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_resmisa(s, 1, 0, false, false, nullptr).bytes;
    return SA_OK;
}

int lisa_score_topk(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                    int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                    void* stream) {
    int rc = check_resmisa(s, 1, 0);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    return run_resmisa(q, w, keys, s, 1, 0, nullptr, nullptr, out_idx, out_score, ws, ws_bytes,
                       stream);
}

int resmisa_route_ws(const sa_shape* s, int32_t block, int32_t r, int32_t extrema_given,
                     size_t* ws_bytes) {
    int rc = check_resmisa(s, block, r);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_resmisa(s, block, r, extrema_given != 0, r > 0 && any_partial(s, block),
                             nullptr)
                    .bytes;
    return SA_OK;
}

int resmisa_route(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                  int32_t block, int32_t r, const uint16_t* extrema, int32_t* out_heads,
                  int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_resmisa(s, block, r);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    return run_resmisa(q, w, keys, s, block, r, extrema, r > 0 ? out_heads : nullptr, out_idx,
                       out_score, ws, ws_bytes, stream);
}

int sa_block_extrema(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t block,
                     uint16_t* out, void* stream) {
    if (!keys || !out) return fail(SA_EINVAL, "keys and out must be non-NULL");
    if (batch < 1 || L < 1 || block < 1) return fail(SA_EINVAL, "batch, L and block must be >= 1");
    if (d != sa::kD) return fail(SA_EUNSUPPORTED, "d must be 128");
    hipError_t e = sa::launch_extrema(keys, batch, L, block, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block extrema");
    return SA_OK;
}

// -------------------------------------------------------------- pooling

int sa_pool_blocks(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t block,
                   uint16_t* out, void* stream) {
    if (!keys || !out) return fail(SA_EINVAL, "keys and out must be non-NULL");
    if (batch < 1 || L < 1 || block < 1) return fail(SA_EINVAL, "batch, L, block must be >= 1");
    if (d != sa::kD) return fail(SA_EUNSUPPORTED, "d must be 128");
    hipError_t e = sa::launch_pool(keys, batch, L, block, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pool");
    return SA_OK;
}

int sa_pool_blocks2(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t small,
                    int32_t large, uint16_t* out_small, uint16_t* out_large, void* stream) {
    if (!keys || !out_small || !out_large) return fail(SA_EINVAL, "NULL pointer");
    if (batch < 1 || L < 1 || small < 1 || large < small || large % small != 0)
        return fail(SA_EINVAL, "need batch, L >= 1 and large a multiple of small");
    if (d != sa::kD) return fail(SA_EUNSUPPORTED, "d must be 128");
    hipError_t e = sa::launch_pool2(keys, batch, L, small, large, out_small, out_large,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pool2");
    return SA_OK;
}

// ----------------------------------------------------------------- MISA

// MISA router stage: pooled keys (given, or pooled into pooled_ws), the
// pooled means of cut last blocks (tail != null), the router -> heads
// [rows, h] ascending.
static int route_heads(const uint16_t* q, const float* w, const uint16_t* keys,
                       const sa_shape* s, int block_B, int h, const uint16_t* pooled,
                       uint16_t* pooled_ws, uint16_t* tail, uint8_t* flag, int32_t* heads,
                       hipStream_t st, uint32_t* zero_state = nullptr,
                       const uint8_t* codes = nullptr, const float* kscale = nullptr,
                       uint16_t* qp = nullptr, float* wp = nullptr) {
    const int rows = s->batch * s->T;
    const int nblk = (s->L + block_B - 1) / block_B;
    hipError_t e;
    const uint16_t* reps = pooled;
    if (!reps) {
        e = sa::launch_pool(keys, s->batch, s->L, block_B, pooled_ws, st, codes, kscale);
        if (e != hipSuccess) return hip_fail(e, "pool");
        reps = pooled_ws;
    }
    if (tail) {
        e = sa::launch_tail(keys, (long long)s->L * sa::kD, s->T, s->causal_offset, s->L,
                            block_B, rows, tail, flag, st, codes, kscale);
        if (e != hipSuccess) return hip_fail(e, "tail pool");
    }
    sa::RouterArgs ra{};
    ra.q = q;
    ra.w = w;
    ra.reps = reps;
    ra.seq_stride = (long long)nblk * 2 * sa::kD;
    ra.tail = tail;
    ra.tail_flag = tail ? flag : nullptr;
    ra.T = s->T;
    ra.H = s->H;
    ra.offset = s->causal_offset;
    ra.B = block_B;
    ra.nblk = nblk;
    ra.h = h;
    ra.heads_out = heads;
    ra.E_out = nullptr;
    ra.zero_state = zero_state;
    ra.qp = qp;
    ra.wp = wp;
    e = sa::launch_router(ra, rows, st);
    if (e != hipSuccess) return hip_fail(e, "router");
    return SA_OK;
}

int misa_route_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                  int32_t pooled_given, size_t* ws_bytes) {
    int rc = check_misa(s, block_B, h, k_prime);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_misa(s, block_B, h, k_prime, pooled_given != 0, any_partial(s, block_B),
                          nullptr)
                    .bytes;
    return SA_OK;
}

// MISA over bf16 keys, or over an FP8 cache (codes, kscale; keys null).
static int run_misa(const uint16_t* q, const float* w, const uint16_t* keys, const uint8_t* codes,
                    const float* kscale, const sa_shape* s, int32_t block_B, int32_t h,
                    int32_t k_prime, const uint16_t* pooled, int32_t* out_heads,
                    int32_t* out_pool, int32_t* out_idx, float* out_score, void* ws,
                    size_t ws_bytes, void* stream, int32_t phases = 3) {
    int rc = check_misa(s, block_B, h, k_prime);
    if (rc) return rc;
    if (phases < 1 || phases > 3) return fail(SA_EINVAL, "phases must be 1, 2 or 3");
    const bool partial = any_partial(s, block_B);
    const size_t need = plan_misa(s, block_B, h, k_prime, pooled != nullptr, partial, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    MisaPlan p = plan_misa(s, block_B, h, k_prime, pooled != nullptr, partial, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int rows = s->batch * s->T;
    hipError_t e;
    int32_t* heads = out_heads ? out_heads : p.heads;
    int32_t* pool_idx = k_prime ? (out_pool ? out_pool : p.pool_idx) : nullptr;
    if (phases != 3 && (p.prefill || codes || partial))
        return fail(SA_EUNSUPPORTED,
                    "calls in phases take decode rows on bf16 keys with whole blocks only");
    if (!p.prefill && !codes && !partial) {
        // Decode rows on bf16 keys, no block cut by the causal bound: the
        // routed scan routes each row itself (no router launch).
        const uint16_t* reps = pooled;
        if (!reps && (phases & 1)) {
            e = sa::launch_pool(keys, s->batch, s->L, block_B, p.pooled, st);
            if (e != hipSuccess) return hip_fail(e, "pool");
        }
        if (!reps) reps = p.pooled;
        const int kk = k_prime ? k_prime : s->topk;
        e = run_dense_topk(q, w, keys, s, heads, h, p.scores, p.state, p.cand, kk,
                           k_prime ? pool_idx : out_idx, k_prime ? nullptr : out_score, st,
                           nullptr, nullptr, /*state_zeroed=*/false, nullptr, 0, false, nullptr,
                           nullptr, 0, 0, nullptr, reps, block_B, phases);
        if (e != hipSuccess) return hip_fail(e, "routed scan");
        if (k_prime == 0 || !(phases & 2)) return SA_OK;
    } else {
        rc = route_heads(q, w, keys, s, block_B, h, pooled, p.pooled, partial ? p.tail : nullptr,
                         p.flag, heads, st, p.state, codes, kscale, p.qp, p.wp);
        if (rc) return rc;
    }
    const bool routed_inline = !p.prefill && !codes && !partial;
    if (p.prefill) {
        // The routed score of every legal key is the DSA score of the h
        // routed heads: the fused prefill on their q rows keeps the top-k (or
        // the k' pool) without writing any score row.
        sa::PrefillArgs pa{};
        pa.q = p.qp;
        pa.w = p.wp;
        pa.keys = keys;
        pa.T = s->T;
        pa.H = h;
        pa.L = s->L;
        pa.offset = s->causal_offset;
        pa.k = k_prime ? k_prime : s->topk;
        pa.surv = p.surv;
        pa.cap = surv_cap((long long)s->causal_offset + s->T, pa.k);
        pa.out_idx = k_prime ? pool_idx : out_idx;
        pa.out_score = k_prime ? nullptr : out_score;
        pa.out_stride = k_prime ? k_prime : s->topk;
        e = sa::launch_prefill(pa, rows, st);
        if (e != hipSuccess) return hip_fail(e, "routed prefill");
        if (k_prime == 0) return SA_OK;
    }
    if (k_prime == 0) {
        e = run_dense_topk(q, w, keys, s, heads, h, p.scores, p.state, p.cand, s->topk,
                           out_idx, out_score, st, codes, kscale, /*state_zeroed=*/true);
        if (e != hipSuccess) return hip_fail(e, "routed scan");
        return SA_OK;
    }
    if (!p.prefill && !routed_inline) {
        e = run_dense_topk(q, w, keys, s, heads, h, p.scores, p.state, p.cand, k_prime, pool_idx,
                           nullptr, st, codes, kscale, /*state_zeroed=*/true);
        if (e != hipSuccess) return hip_fail(e, "routed scan");
    }
    sa::GatherArgs ga{};
    ga.q = q;
    ga.w = w;
    ga.keys = keys;
    ga.seq_stride = (long long)s->L * sa::kD;
    ga.list = pool_idx;
    ga.list_len = k_prime;
    ga.bsz = 1;
    ga.ncand = k_prime;
    ga.T = s->T;
    ga.H = s->H;
    ga.L = s->L;
    ga.offset = s->causal_offset;
    ga.out_score = p.list_score;
    ga.out_idx = p.list_idx;
    ga.codes = codes;
    ga.kscale = kscale;
    e = sa::launch_gather(ga, rows, (s->H + 15) / 16, false, st);
    if (e != hipSuccess) return hip_fail(e, "rerank");
    e = run_list_topk(p.list_score, p.list_idx, k_prime, nullptr, k_prime, rows, s->topk,
                      out_idx, out_score, st);
    if (e != hipSuccess) return hip_fail(e, "rerank top-k");
    return SA_OK;
}

int misa_route(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
               int32_t block_B, int32_t h, int32_t k_prime, const uint16_t* pooled,
               int32_t* out_heads, int32_t* out_pool, int32_t* out_idx, float* out_score,
               void* ws, size_t ws_bytes, void* stream) {
    int rc = check_misa(s, block_B, h, k_prime);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    return run_misa(q, w, keys, nullptr, nullptr, s, block_B, h, k_prime, pooled, out_heads,
                    out_pool, out_idx, out_score, ws, ws_bytes, stream);
}

int misa_route_phase(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                     int32_t block_B, int32_t h, int32_t k_prime, const uint16_t* pooled,
                     int32_t* out_heads, int32_t* out_pool, int32_t* out_idx, float* out_score,
                     void* ws, size_t ws_bytes, int32_t phases, void* stream) {
    int rc = check_misa(s, block_B, h, k_prime);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    return run_misa(q, w, keys, nullptr, nullptr, s, block_B, h, k_prime, pooled, out_heads,
                    out_pool, out_idx, out_score, ws, ws_bytes, stream, phases);
}

int misa_route_fp8_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                      int32_t pooled_given, size_t* ws_bytes) {
    if (s && s->T >= kPrefillMinT)
        return fail(SA_EUNSUPPORTED, "FP8 keys: MISA takes decode-style rows only (T < 16)");
    return misa_route_ws(s, block_B, h, k_prime, pooled_given, ws_bytes);
}

int misa_route_fp8(const uint16_t* q, const float* w, const uint8_t* codes, const float* scales,
                   const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                   const uint16_t* pooled, int32_t* out_heads, int32_t* out_pool,
                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_misa(s, block_B, h, k_prime);
    if (rc) return rc;
    if (s->T >= kPrefillMinT)
        return fail(SA_EUNSUPPORTED, "FP8 keys: MISA takes decode-style rows only (T < 16)");
    if (!q || !w || !codes || !scales || !out_idx)
        return fail(SA_EINVAL, "q, w, codes, scales and out_idx must be non-NULL");
    return run_misa(q, w, nullptr, codes, scales, s, block_B, h, k_prime, pooled, out_heads,
                    out_pool, out_idx, out_score, ws, ws_bytes, stream);
}

// ----------------------------------------------------------------- HISA

int hisa_coarse_fine_ws(const sa_shape* s, int32_t block_b, int32_t r, int32_t reps_given,
                        size_t* ws_bytes) {
    int rc = check_hisa(s, block_b, r);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_hisa(s, block_b, r, reps_given != 0, any_partial(s, block_b), nullptr).bytes;
    return SA_OK;
}

// HISA stages: block reps (given, or pooled into the plan), the means of cut
// last blocks, block scores (over `heads` [rows, hsel] when given: the MISA x
// HISA composition, else every head), top-r blocks, every-head rescoring of
// their legal tokens, token top-k.
static int hisa_stages(const uint16_t* q, const float* w, const uint16_t* keys,
                       const sa_shape* s, int block_b, int r, const uint16_t* reps,
                       const HisaPlan& p, bool partial, const int32_t* heads, int hsel,
                       int32_t* out_blocks, int32_t* out_idx, float* out_score, hipStream_t st,
                       const uint8_t* codes = nullptr, const float* kscale = nullptr) {
    const int rows = s->batch * s->T;
    const int nblk = (s->L + block_b - 1) / block_b;
    hipError_t e;
    const uint16_t* rp = reps;
    if (!rp) {
        e = sa::launch_pool(keys, s->batch, s->L, block_b, p.reps, st, codes, kscale);
        if (e != hipSuccess) return hip_fail(e, "pool");
        rp = p.reps;
    }
    if (partial) {
        e = sa::launch_tail(keys, (long long)s->L * sa::kD, s->T, s->causal_offset, s->L,
                            block_b, rows, p.tail, p.flag, st, codes, kscale);
        if (e != hipSuccess) return hip_fail(e, "tail pool");
    }
    // Coarse stage: block scores with the indexer formula (routed heads or all).
    sa::ScanArgs a{};
    a.q = q;
    a.w = w;
    a.keys = rp;
    a.seq_stride = (long long)nblk * 2 * sa::kD;
    a.tail = p.tail;
    a.tail_flag = p.flag;
    a.T = s->T;
    a.H = s->H;
    a.offset = s->causal_offset;
    a.len_div = block_b;
    a.len_cap = nblk;
    a.chunk = sa::scan_chunk(8, rows, nblk);
    a.scores = p.bscores;
    a.score_stride = nblk;
    a.heads = heads;
    a.hsel = hsel;
    e = sa::launch_scan(a, rows, ((heads ? hsel : s->H) + 15) / 16, 8, heads != nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "block scores");
    int32_t* blocks = out_blocks ? out_blocks : p.blocks;
    sa::TopkArgs t{};
    t.dense = p.bscores;
    t.dense_stride = nblk;
    t.T = s->T;
    t.offset = s->causal_offset;
    t.len_div = block_b;
    t.len_cap = nblk;
    t.k = r;
    t.out_idx = blocks;
    t.out_score = nullptr;
    t.out_stride = r;
    e = sa::launch_topk(t, rows, st);
    if (e != hipSuccess) return hip_fail(e, "block top-r");
    // Fine stage: exact scores on the legal tokens of the kept blocks.
    sa::GatherArgs ga{};
    ga.q = q;
    ga.w = w;
    ga.keys = keys;
    ga.seq_stride = (long long)s->L * sa::kD;
    ga.list = blocks;
    ga.list_len = r;
    ga.bsz = block_b;
    ga.ncand = r * block_b;
    ga.T = s->T;
    ga.H = s->H;
    ga.L = s->L;
    ga.offset = s->causal_offset;
    ga.out_score = p.list_score;
    ga.out_idx = p.list_idx;
    ga.codes = codes;
    ga.kscale = kscale;
    e = sa::launch_gather(ga, rows, (s->H + 15) / 16, true, st);
    if (e != hipSuccess) return hip_fail(e, "fine rescore");
    e = run_list_topk(p.list_score, p.list_idx, (long long)r * block_b, nullptr, r * block_b,
                      rows, s->topk, out_idx, out_score, st);
    if (e != hipSuccess) return hip_fail(e, "fine top-k");
    return SA_OK;
}

int hisa_coarse_fine(const uint16_t* q, const float* w, const uint16_t* keys,
                     const sa_shape* s, int32_t block_b, int32_t r, const uint16_t* reps,
                     int32_t* out_blocks, int32_t* out_idx, float* out_score, void* ws,
                     size_t ws_bytes, void* stream) {
    int rc = check_hisa(s, block_b, r);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    const bool partial = any_partial(s, block_b);
    const size_t need = plan_hisa(s, block_b, r, reps != nullptr, partial, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    HisaPlan p = plan_hisa(s, block_b, r, reps != nullptr, partial, base);
    return hisa_stages(q, w, keys, s, block_b, r, reps, p, partial, nullptr, 0, out_blocks,
                       out_idx, out_score, static_cast<hipStream_t>(stream));
}

int hisa_coarse_fine_fp8_ws(const sa_shape* s, int32_t block_b, int32_t r, int32_t reps_given,
                            size_t* ws_bytes) {
    return hisa_coarse_fine_ws(s, block_b, r, reps_given, ws_bytes);
}

int hisa_coarse_fine_fp8(const uint16_t* q, const float* w, const uint8_t* codes,
                         const float* scales, const sa_shape* s, int32_t block_b, int32_t r,
                         const uint16_t* reps, int32_t* out_blocks, int32_t* out_idx,
                         float* out_score, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_hisa(s, block_b, r);
    if (rc) return rc;
    if (!q || !w || !codes || !scales || !out_idx)
        return fail(SA_EINVAL, "q, w, codes, scales and out_idx must be non-NULL");
    const bool partial = any_partial(s, block_b);
    const size_t need = plan_hisa(s, block_b, r, reps != nullptr, partial, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    HisaPlan p = plan_hisa(s, block_b, r, reps != nullptr, partial, base);
    return hisa_stages(q, w, nullptr, s, block_b, r, reps, p, partial, nullptr, 0, out_blocks,
                       out_idx, out_score, static_cast<hipStream_t>(stream), codes, scales);
}

// ------------------------------------------------------------ MISA x HISA

struct MisaHisaPlan {
    uint16_t* pooled;
    uint16_t* tail;
    uint8_t* flag;
    int32_t* heads;
    HisaPlan hisa;
    size_t bytes;
};

static MisaHisaPlan plan_misa_hisa(const sa_shape* s, int B, int h, int b, int r,
                                   bool pooled_given, bool reps_given, void* ws) {
    MisaHisaPlan p{};
    Carve cv(ws);
    const long long rows = (long long)s->batch * s->T;
    const long long nblk = (s->L + B - 1) / B;
    if (!pooled_given) p.pooled = cv.take<uint16_t>(s->batch * nblk * 2 * sa::kD);
    if (any_partial(s, B)) {
        p.tail = cv.take<uint16_t>(rows * 2 * sa::kD);
        p.flag = cv.take<uint8_t>(rows);
    }
    p.heads = cv.take<int32_t>(rows * h);
    const size_t off = (cv.off + 255) & ~size_t(255);
    p.hisa = plan_hisa(s, b, r, reps_given, any_partial(s, b),
                       ws ? static_cast<char*>(ws) + off : nullptr);
    p.bytes = off + p.hisa.bytes;
    return p;
}

int misa_hisa_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t block_b, int32_t r,
                 int32_t pooled_given, int32_t reps_given, size_t* ws_bytes) {
    int rc = check_misa(s, block_B, h, 0);
    if (rc) return rc;
    rc = check_hisa(s, block_b, r);
    if (rc) return rc;
    if (!ws_bytes) return fail(SA_EINVAL, "ws_bytes is NULL");
    *ws_bytes = plan_misa_hisa(s, block_B, h, block_b, r, pooled_given != 0, reps_given != 0,
                               nullptr)
                    .bytes;
    return SA_OK;
}

int misa_hisa(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
              int32_t block_B, int32_t h, int32_t block_b, int32_t r, const uint16_t* pooled,
              const uint16_t* reps, int32_t* out_heads, int32_t* out_blocks, int32_t* out_idx,
              float* out_score, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_misa(s, block_B, h, 0);
    if (rc) return rc;
    rc = check_hisa(s, block_b, r);
    if (rc) return rc;
    rc = check_ptrs(q, w, keys, out_idx);
    if (rc) return rc;
    const size_t need =
        plan_misa_hisa(s, block_B, h, block_b, r, pooled != nullptr, reps != nullptr, nullptr).bytes;
    if (!ws || ws_bytes < need) return fail(SA_EWORKSPACE, "workspace too small");
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    MisaHisaPlan p =
        plan_misa_hisa(s, block_B, h, block_b, r, pooled != nullptr, reps != nullptr, base);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* heads = out_heads ? out_heads : p.heads;
    rc = route_heads(q, w, keys, s, block_B, h, pooled, p.pooled, p.tail, p.flag, heads, st);
    if (rc) return rc;
    return hisa_stages(q, w, keys, s, block_b, r, reps, p.hisa, any_partial(s, block_b), heads, h,
                       out_blocks, out_idx, out_score, st);
}

}  // extern "C"
