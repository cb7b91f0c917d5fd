// Host runtime of the looped-KV library: configuration checks, KV-store layout,
// workspace layout and the prefill / decode loop drivers behind the C ABI.
//
// Loop structure: embed -> P prelude layers -> K passes of the R shared layers,
// the loop embedding added before each pass -> Q coda layers -> final RMSNorm
// (FlashLoop walk-through, discosf.com, sections 3.1 and 4.1).  KV modes
// per_loop / last_loop: Looped Transformer tutorial (aiboss88.com, step 4).
// Lazy mode: FlashLoop abstract (arxivdaily.com) -- token-sparse loop updates,
// sparse attention over stable key columns, quantized KV residuals.
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/looped_kv.h"
#include "lk_kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

#define LK_HIP(call)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) return fail(LK_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

#define LK_TRY(call)          \
    do {                      \
        int r_ = (call);      \
        if (r_ != LK_OK) return r_; \
    } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Loop k >= 2 recomputes every token when the refresh period divides k - 1.
bool refresh_loop(const lk_lazy_cfg& z, int k) { return z.refresh_every > 0 && (k - 1) % z.refresh_every == 0; }

int n_selected(double rho, int T) {
    if (T <= 0) return 0;
    long long n = (long long)std::ceil(rho * (double)T - 1e-9);
    if (n < 1) n = 1;
    if (n > T) n = T;
    return (int)n;
}

// Columns per split and the split-count ceiling of the row-attention kernel.
constexpr int kRowChunk = 256;
constexpr int kMaxSplits = 256;
// Rows per split of the two-segment decode attention (stable-column cache, window ring).
constexpr int kSegChunk = 128;

// Dense decode attention over ncol keys of `pairs` (sequence, KV head) pairs: one
// workgroup per (pair, chunk), about 768 workgroups (three per CU; longer chunks keep
// each wave streaming longer).
int decode_dense_chunk(long long pairs, long long ncol) {
    const long long want = (ncol * pairs + 767) / 768;
    int ch = (int)std::max(128LL, (want + 127) / 128 * 128);
    while ((ncol + ch - 1) / ch > kMaxSplits) ch *= 2;
    return ch;
}

}  // namespace

// Kernel classes that can be bracketed with HIP events (instrumentation).
enum TimedClass { TC_NONE = -1, TC_ATTN_DECODE_DENSE = 0, TC_ATTN_DECODE_SPARSE, TC_ATTN_PREFILL,
                  TC_COLUMN_MASS, TC_ATTN_PREFILL_SPARSE, TC_GEMM_DECODE, TC_GEMM_PREFILL, TC_COUNT };
static const char* kTimedNames[TC_COUNT] = {"attn_decode_dense", "attn_decode_sparse", "attn_prefill",
                                            "column_mass", "attn_prefill_sparse", "gemm_decode",
                                            "gemm_prefill"};

struct EventTimer {
    unsigned mask = 0;  // bit c: kernel class c is timed
    int per_call = 0;   // launches of each class timed per prefill / decode call (0: all)
    int in_call[TC_COUNT] = {};  // launches of each class seen in the current call
    std::vector<hipEvent_t> pool;  // pairs (start, end), one per timed launch
    std::vector<int> pair_cls;     // class of each pair
    size_t used = 0;
    bool wants(int cls) {
        if (cls < 0 || !((mask >> cls) & 1u)) return false;
        return per_call == 0 || in_call[cls]++ < per_call;
    }
    void new_call() {
        for (int& c : in_call) c = 0;
    }
    hipError_t mark(hipStream_t st) {
        if (used == pool.size()) {
            hipEvent_t e;
            hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) return r;
            pool.push_back(e);
        }
        return hipEventRecord(pool[used++], st);
    }
    hipError_t begin(hipStream_t st, int cls) {
        if (pair_cls.size() < used / 2 + 1) pair_cls.resize(used / 2 + 1);
        pair_cls[used / 2] = cls;
        return mark(st);
    }
    ~EventTimer() {
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    }
};

// A decode step prepared for replay: captured HIP graphs, cut around every launch
// of the timed kernel class (those are launched directly, between two recorded
// events, so that their duration is measured on the stream), plus the key it was
// prepared for.  With timing off the step is one graph.
struct DecodeGraph {
    struct Seg {
        hipGraphExec_t exec = nullptr;           // a captured run of launches, or
        std::function<hipError_t()> direct;      // one timed launch
        int cls = -1;                            // its kernel class
    };
    std::vector<Seg> segs;
    const void* store = nullptr;
    const void* ws = nullptr;
    hipStream_t stream = nullptr;
    long long timer_mask = -1;
    int timer_per_call = -1;
    int keep_codes = 0;
    void reset() {
        for (Seg& g : segs)
            if (g.exec) (void)hipGraphExecDestroy(g.exec);
        segs.clear();
        store = ws = nullptr;
        stream = nullptr;
        timer_mask = -1;
    }
    ~DecodeGraph() { reset(); }
};

struct lk_handle {
    lk_model_cfg c;
    lk_lazy_cfg z;
    EventTimer timer;
    DecodeGraph graph;
    DecodeGraph* building = nullptr;  // set while a decode step is being captured
    int use_graphs = 1;
    // Decode copy of the layer projections in the lane-packed operand order, in a
    // caller-owned buffer given by lk_set_decode_weights (nullptr: decode multiplies by
    // the row-major weights).
    struct Packed {
        const u16 *wqkv, *wo, *w_in, *w_down;
    };
    std::vector<Packed> PL;
    void* pk_buf = nullptr;
    const u16 *tok, *lemb, *fnorm;
    std::vector<lk_layer_weights> L;
    double inv_freq[64];
    int qkv_w() const { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }
    int G() const { return c.n_heads / c.n_kv_heads; }
    bool lazy() const { return z.mode == LK_MODE_LAZY; }
};

struct StoreLayout {
    size_t dense, loop_rows, base, base_sc, res, res_sc, slot, cols, state, scache, total;
    long long slots;
    int n_sel, n_cols;
    int ncs;                 // rows per (b, g) of the stable-column cache (n_cols rounded up to 128)
    int wr;                  // rows per (b, g) of the window ring (window + 16 rounded up to 128)
    int ck0;                 // first cached loop: 2, or 1 with difference-corrected attention
    size_t scache_bytes;     // stable-column cache and window rings together
    long long res_row_b;
};

struct lk_kv_store {
    lk_handle* h;
    int B, Tp, Tmax, t;
    int Tpad;  // row stride: Tmax rounded up to a multiple of 8
    bool prefilled;
    StoreLayout lay;
    char* buf;
    const int32_t* f_tok;
    const int32_t* f_cols;
    int keep_codes;
    int K;  // loops the store runs (<= the model's n_loops)
};

namespace {

// Positions per (sequence, KV head) are padded to a multiple of 8: V rows are
// stored in blocks of 8 interleaved keys.
inline int pad8(int t) { return (t + 7) / 8 * 8; }

StoreLayout store_layout(const lk_handle* h, int B, int Tp, int Tmax) {
    const lk_model_cfg& c = h->c;
    StoreLayout s{};
    const long long hd = c.head_dim, Hkv = c.n_kv_heads;
    const int Tpad = pad8(Tmax);
    const long long kvrows = (long long)B * Hkv * Tpad;  // rows of one K or V region of a layer
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    s.dense = take((size_t)(c.n_prelude + c.n_coda) * 2 * kvrows * hd * 2);
    s.loop_rows = s.base = s.base_sc = s.res = s.res_sc = s.slot = s.cols = off;
    s.slots = 0;
    s.n_sel = 0;
    s.n_cols = 0;
    s.res_row_b = 0;
    if (h->z.mode == LK_MODE_PER_LOOP) {
        s.loop_rows = take((size_t)c.n_loops * c.n_shared * 2 * kvrows * hd * 2);
    } else if (h->z.mode == LK_MODE_LAST_LOOP) {
        s.loop_rows = take((size_t)c.n_shared * 2 * kvrows * hd * 2);
    } else {
        const int bb = h->z.base_bits == 16 ? 2 : 1;
        s.base = take((size_t)c.n_shared * 2 * kvrows * hd * bb);
        s.base_sc = take(h->z.base_bits == 16 ? 0 : (size_t)c.n_shared * 2 * kvrows * (hd / 32) * 2);
        s.n_sel = n_selected(h->z.rho, Tp);
        int most = s.n_sel;  // the most prompt rows a loop stores
        for (int k = 2; k <= c.n_loops; ++k)
            if (refresh_loop(h->z, k)) most = Tp;
        s.slots = (long long)most + (Tmax - Tp);
        s.res_row_b = h->z.res_bits == 16 ? hd * 2 : hd * h->z.res_bits / 8;
        const long long res_rows = (long long)(c.n_loops - 1) * c.n_shared * 2 * B * Hkv * s.slots;
        s.res = take((size_t)res_rows * s.res_row_b);
        s.res_sc = take(h->z.res_bits == 16 ? 0 : (size_t)res_rows * (hd / 32) * 2);
        s.slot = take((size_t)(c.n_loops - 1) * B * Tpad * 4);
        s.n_cols = h->z.top_s < Tp ? h->z.top_s : Tp;
        s.cols = take((size_t)c.n_shared * B * Hkv * s.n_cols * 4);
    }
    s.state = take(64);  // int32 decode position t (device copy of the store length)
    // Decode cache: for every loop k >= ck0 and shared layer r, the float16 loop-k
    // reconstruction of the stable columns S (fixed once prefill has run), K rows
    // [B][Hkv][ncs][hd] then 8-key-interleaved V [B][Hkv][ncs/8][hd][8].
    // Then the window rings: per loop k >= ck0 and shared layer r, the float16 loop-k
    // reconstruction of the last wr positions (position p at row p % wr), K then V as
    // above; prefill fills them, every decode step writes its own row.  ck0 = 2, or 1
    // when difference-corrected attention also takes a sparse term at loop 1.
    s.ncs = s.wr = 0;
    s.ck0 = h->z.diff_attn ? 1 : 2;
    s.scache_bytes = 0;
    s.scache = off;
    if (h->z.mode == LK_MODE_LAZY && c.n_loops >= 2) {
        s.ncs = (s.n_cols + 127) / 128 * 128;
        s.wr = (h->z.window + 16 + 127) / 128 * 128;
        s.scache_bytes = (size_t)(c.n_loops + 1 - s.ck0) * c.n_shared * 2 * B * Hkv * ((size_t)s.ncs + s.wr) * hd * 2;
        s.scache = take(s.scache_bytes);
    }
    s.total = off;
    return s;
}

// Prompt rows loop k >= 2 recomputes and stores: every one at a refresh loop, else n.
int loop_rows(const lk_kv_store* s, int k) { return refresh_loop(s->h->z, k) ? s->Tp : s->lay.n_sel; }

// Bytes of stored data at length t (closed form, no alignment padding).
void store_bytes(const lk_kv_store* s, size_t* shared, size_t* total) {
    const lk_handle* h = s->h;
    const lk_model_cfg& c = h->c;
    const long long E = 2LL * c.n_kv_heads * c.head_dim;
    const long long t = s->t;
    const long long B = s->B;
    const long long dense = (long long)(c.n_prelude + c.n_coda) * B * t * E * 2;
    long long sh = 0;
    auto rowb = [&](long long n, int bits) -> long long {
        return bits == 16 ? 2 * n : n * bits / 8 + (n / 32) * 2;
    };
    if (h->z.mode == LK_MODE_PER_LOOP) {
        sh = (long long)c.n_shared * s->K * B * t * E * 2;
    } else if (h->z.mode == LK_MODE_LAST_LOOP) {
        sh = (long long)c.n_shared * B * t * E * 2;
    } else if (t > 0) {
        long long stored = 0;  // rows per sequence over loops 2..K: recomputed prompt rows + decoded
        for (int k = 2; k <= s->K; ++k) stored += loop_rows(s, k) + (t - s->Tp);
        sh = (long long)c.n_shared * B * t * rowb(E, h->z.base_bits) +
             (long long)c.n_shared * B * stored * rowb(E, h->z.res_bits) +
             (long long)(s->K - 1) * B * t * 4 + (long long)c.n_shared * B * c.n_kv_heads * s->lay.n_cols * 4;
    }
    *shared = (size_t)sh;
    *total = (size_t)(sh + dense);
}

// K/V row pointers ------------------------------------------------------------
long long kv_region_elems(const lk_kv_store* s) {
    return (long long)s->B * s->h->c.n_kv_heads * s->Tpad * s->h->c.head_dim;
}

KVLayer plain_layer(const lk_kv_store* s, u16* k_rows, u16* v_rows) {
    KVLayer L{};
    const lk_model_cfg& c = s->h->c;
    L.lazy = 0;
    L.B = s->B;
    L.Hkv = c.n_kv_heads;
    L.hd = c.head_dim;
    L.Tmax = s->Tpad;
    L.base_bits = 16;
    L.res_bits = 16;
    L.n_loops = c.n_loops;
    L.base[0] = k_rows;
    L.base[1] = v_rows;
    return L;
}

KVLayer dense_layer(const lk_kv_store* s, int ci) {
    u16* base = (u16*)(s->buf + s->lay.dense);
    const long long n = kv_region_elems(s);
    return plain_layer(s, base + (2LL * ci) * n, base + (2LL * ci + 1) * n);
}

KVLayer loop_layer(const lk_kv_store* s, int k, int r) {
    u16* base = (u16*)(s->buf + s->lay.loop_rows);
    const long long n = kv_region_elems(s);
    const long long idx = s->h->z.mode == LK_MODE_PER_LOOP ? ((long long)(k - 1) * s->h->c.n_shared + r) : r;
    return plain_layer(s, base + (2 * idx) * n, base + (2 * idx + 1) * n);
}

KVLayer lazy_layer(const lk_kv_store* s, int r) {
    const lk_handle* h = s->h;
    const lk_model_cfg& c = h->c;
    KVLayer L{};
    L.lazy = 1;
    L.B = s->B;
    L.Hkv = c.n_kv_heads;
    L.hd = c.head_dim;
    L.Tmax = s->Tpad;
    L.slots = s->lay.slots;
    L.base_bits = h->z.base_bits;
    L.res_bits = h->z.res_bits;
    L.n_loops = c.n_loops;
    const long long n = kv_region_elems(s);
    const long long bb = h->z.base_bits == 16 ? 2 : 1;
    const long long nsc = n / c.head_dim * (c.head_dim / 32);
    for (int kv = 0; kv < 2; ++kv) {
        L.base[kv] = s->buf + s->lay.base + (2LL * r + kv) * n * bb;
        L.base_scale[kv] = h->z.base_bits == 16 ? nullptr : (const u16*)(s->buf + s->lay.base_sc) + (2LL * r + kv) * nsc;
    }
    const long long rows = (long long)s->B * c.n_kv_heads * s->lay.slots;  // rows of one (k, r, kv) region
    for (int kk = 2; kk <= c.n_loops; ++kk)
        for (int kv = 0; kv < 2; ++kv) {
            const long long reg = ((long long)(kk - 2) * c.n_shared + r) * 2 + kv;
            L.res[kk - 2][kv] = s->buf + s->lay.res + reg * rows * s->lay.res_row_b;
            L.res_scale[kk - 2][kv] =
                h->z.res_bits == 16 ? nullptr : (const u16*)(s->buf + s->lay.res_sc) + reg * rows * (c.head_dim / 32);
        }
    L.slot = (const int32_t*)(s->buf + s->lay.slot);
    return L;
}

int32_t* slot_map(const lk_kv_store* s, int k) {
    return (int32_t*)(s->buf + s->lay.slot) + (long long)(k - 2) * s->B * s->Tpad;
}
int32_t* dev_pos(const lk_kv_store* s) { return (int32_t*)(s->buf + s->lay.state); }
// The store's float16-range flag (KVWrite::range_flag), beside the decode position.
uint32_t* range_flag(const lk_kv_store* s) { return (uint32_t*)(s->buf + s->lay.state + 4); }

// Stable-column cache (ring == false) or window ring (ring == true) of loop k >= ck0,
// shared layer r, as float16 plain rows.
KVLayer scache_layer(const lk_kv_store* s, int k, int r, bool ring = false) {
    const lk_model_cfg& c = s->h->c;
    const int rows = ring ? s->lay.wr : s->lay.ncs;
    const int k0 = s->lay.ck0;
    const size_t one = (size_t)s->B * c.n_kv_heads * rows * c.head_dim * 2;  // K or V of one (k, r)
    size_t off = s->lay.scache + ((size_t)(k - k0) * c.n_shared + r) * 2 * one;
    if (ring)
        off += (size_t)(c.n_loops + 1 - k0) * c.n_shared * 2 * s->B * c.n_kv_heads * s->lay.ncs * c.head_dim * 2;
    char* base = s->buf + off;
    KVLayer L{};
    L.lazy = 0;
    L.f16 = 1;
    L.B = s->B;
    L.Hkv = c.n_kv_heads;
    L.hd = c.head_dim;
    L.Tmax = rows;
    L.base_bits = 16;
    L.res_bits = 16;
    L.n_loops = c.n_loops;
    L.base[0] = base;
    L.base[1] = base + one;
    return L;
}

int32_t* col_sets(const lk_kv_store* s, int r) {
    return (int32_t*)(s->buf + s->lay.cols) + (long long)r * s->B * s->h->c.n_kv_heads * s->lay.n_cols;
}

// Workspace -------------------------------------------------------------------
struct WS {
    float *h, *h0, *xc, *qkv, *lse, *mass, *keys, *part;
    u16 *xn, *q, *att, *act;
    int32_t* sel;
    int32_t* ids;      // decode: the step's token ids (fixed address for graph replay)
    float* out;        // decode: the step's output rows
    float* ps;         // decode: per-workgroup row sums of x^2 for the next RMSNorm ([d/8][8])
    float* tokrec;     // decode, lazy: float32 K/V reconstruction of the step's rows [R][B][2][Hkv][hd]
    float* rope;       // decode: cos and sin of the step's position, [hd/2][2]
    float* rope_tab;   // prefill: cos and sin of every prompt position, [T][hd/2][2]
    u16 *frk, *frv;    // prefill, lazy loops >= 2 (hd 128): float16 loop-k K/V at every prompt position
    int fr_cap;        // rows per (b, g) of frk / frv (T rounded up to 64; 0: none)
    int rope_rows;     // prefill: positions in rope_tab (T; 0: none)
    // difference-corrected sparse attention: each row's loop-1 dense minus sparse output
    // per shared layer; prefill float16 [R][B][T][H hd], decode float32 [R][B][H hd]
    u16* dprompt;
    float* dstep;
    // decode-time loop skipping: h_{k-2} per sequence (the final state of a token that
    // left), h_{k-1} saved by the last layer of a loop, and the still-in-the-loops flags
    float *sk_prev, *sk_save;
    int32_t *sk_act, *sk_live;  // flags per sequence; how many are still in the loops
    size_t total;
    long long part_floats;
};

WS ws_layout(const lk_handle* hd_, int B, int T, char* base) {
    const lk_model_cfg& c = hd_->c;
    const long long M = (long long)B * T;
    const long long d = c.d_model;
    long long n = T;  // rows a loop >= 2 recomputes (the most over the loops)
    if (hd_->lazy()) {
        n = n_selected(hd_->z.rho, T);
        for (int k = 2; k <= c.n_loops; ++k)
            if (refresh_loop(hd_->z, k)) n = T;
    }
    const long long Hhd = (long long)c.n_heads * c.head_dim;
    WS w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return base ? (void*)(base + o) : nullptr;
    };
    w.h = (float*)take(M * d * 4);
    w.h0 = (float*)take(hd_->lazy() || c.input_reinject ? M * d * 4 : 0);
    w.xc = (float*)take(hd_->lazy() ? (long long)B * n * d * 4 : 0);
    // 16-bit operands of the decode products are lane-packed over 8 rows (at least 8 rows)
    const long long M8 = M < 8 ? 8 : M;
    w.xn = (u16*)take(M8 * d * 2);
    w.qkv = (float*)take(M * hd_->qkv_w() * 4);
    w.q = (u16*)take(M * Hhd * 2);
    w.att = (u16*)take(M8 * Hhd * 2);
    w.act = (u16*)take(M8 * (long long)c.ffn_dim * 2);
    w.lse = (float*)take(M * c.n_heads * 4);
    w.mass = (float*)take(hd_->lazy() ? M * c.n_kv_heads * 4 : 0);
    w.keys = (float*)take(hd_->lazy() ? M * 4 : 0);
    const bool diff = hd_->lazy() && hd_->z.diff_attn && c.n_loops >= 2;
    // the loop-1 sparse term of the difference correction runs over every prompt row
    const long long n_att = diff ? std::max(n, (long long)T) : n;
    w.sel = (int32_t*)take(hd_->lazy() ? (long long)B * n_att * 4 : 0);
    // row-attention partials: decode rows use up to kMaxSplits splits; token-sparse
    // prefill rows need ceil((columns + window) / chunk) splits.
    long long pf = (long long)B * c.n_heads * kMaxSplits * (c.head_dim + 2);
    const bool fr_path = hd_->lazy() && T > 1 && c.n_loops >= 2 && c.head_dim == 128;
    if (hd_->lazy() && T > 1) {
        const long long ncol = std::min((long long)std::min(hd_->z.top_s, T) + hd_->z.window, (long long)T);
        const long long sp = (ncol + kRowChunk - 1) / kRowChunk;
        // the split-row kernels take the loop-1 sparse term when the float16 path does not
        const long long rows = fr_path ? n : n_att;
        pf = std::max(pf, (long long)B * rows * c.n_heads * sp * (c.head_dim + 2));
    }
    w.part_floats = pf;
    w.part = (float*)take(pf * 4);
    w.ids = (int32_t*)take((long long)B * 4);
    w.ps = (float*)take((d / 8 + 1) * 8 * 4);
    w.tokrec = (float*)take(hd_->lazy() && T == 1 ? (long long)c.n_shared * B * 2 * c.n_kv_heads * c.head_dim * 4 : 0);
    w.fr_cap = fr_path ? (T + 63) / 64 * 64 : 0;
    const long long fr_elems = (long long)B * c.n_kv_heads * w.fr_cap * c.head_dim;
    w.frk = (u16*)take(fr_elems * 2);
    w.frv = (u16*)take(fr_elems * 2);
    w.out = (float*)take((long long)B * d * 4);
    w.rope = (float*)take(T == 1 ? (long long)c.head_dim * 4 : 0);
    w.rope_tab = (float*)take(T > 1 ? (long long)T * c.head_dim * 4 : 0);
    w.rope_rows = T > 1 ? T : 0;
    w.dprompt = (u16*)take(diff ? (long long)c.n_shared * M * Hhd * 2 : 0);
    w.dstep = (float*)take(diff && T == 1 ? (long long)c.n_shared * B * Hhd * 4 : 0);
    const bool skip = hd_->lazy() && hd_->z.skip_tau > 0.f && c.n_loops >= 2 && T == 1;
    w.sk_prev = (float*)take(skip ? (long long)B * d * 4 : 0);
    w.sk_save = (float*)take(skip ? (long long)B * d * 4 : 0);
    w.sk_act = (int32_t*)take(skip ? (long long)B * 4 : 0);
    w.sk_live = (int32_t*)take(skip ? 4 : 0);
    w.total = off;
    return w;
}

int check_cfg(const lk_model_cfg* c, const lk_lazy_cfg* z) {
    if (!c || !z) return fail(LK_ERR_INVALID_ARG, "null config");
    if (c->vocab < 1 || c->d_model < 64 || c->n_heads < 1 || c->n_kv_heads < 1 || c->ffn_dim < 64)
        return fail(LK_ERR_INVALID_ARG, "bad model sizes");
    if (c->n_prelude < 0 || c->n_coda < 0 || c->n_shared < 1 || c->n_loops < 1)
        return fail(LK_ERR_INVALID_ARG, "bad layer counts");
    if (c->n_loops > LK_MAX_LOOPS + 1) return fail(LK_ERR_UNSUPPORTED, "at most 17 loops");
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
        return fail(LK_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
    if (c->n_heads % c->n_kv_heads) return fail(LK_ERR_INVALID_ARG, "n_heads % n_kv_heads != 0");
    const int G = c->n_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(LK_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
    if (c->d_model % 64 || c->ffn_dim % 64) return fail(LK_ERR_UNSUPPORTED, "d_model and ffn_dim must be multiples of 64");
    if ((c->n_heads * c->head_dim) % 64) return fail(LK_ERR_UNSUPPORTED, "n_heads * head_dim must be a multiple of 64");
    if (c->n_kv_heads * c->head_dim > 4096) return fail(LK_ERR_UNSUPPORTED, "n_kv_heads * head_dim > 4096");
    if (c->ffn_act != LK_ACT_GELU && c->ffn_act != LK_ACT_SWIGLU) return fail(LK_ERR_INVALID_ARG, "bad ffn_act");
    if (c->input_reinject != 0 && c->input_reinject != 1) return fail(LK_ERR_INVALID_ARG, "input_reinject must be 0 or 1");
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(LK_ERR_INVALID_ARG, "bad eps / theta");
    if (z->mode != LK_MODE_PER_LOOP && z->mode != LK_MODE_LAST_LOOP && z->mode != LK_MODE_LAZY)
        return fail(LK_ERR_INVALID_ARG, "bad mode");
    if (z->mode == LK_MODE_LAZY) {
        if (!(z->rho > 0.0 && z->rho <= 1.0)) return fail(LK_ERR_INVALID_ARG, "rho must be in (0, 1]");
        if (z->top_s < 1 || z->window < 1) return fail(LK_ERR_INVALID_ARG, "top_s and window must be >= 1");
        if (z->base_bits != 16 && z->base_bits != 8) return fail(LK_ERR_INVALID_ARG, "base_bits must be 16 or 8");
        if (z->res_bits != 16 && z->res_bits != 8 && z->res_bits != 4)
            return fail(LK_ERR_INVALID_ARG, "res_bits must be 16, 8 or 4");
        if (z->group != 32) return fail(LK_ERR_UNSUPPORTED, "group must be 32");
        if (z->stale_keys != 0 && z->stale_keys != 1) return fail(LK_ERR_INVALID_ARG, "stale_keys must be 0 or 1");
        if (z->diff_attn != 0 && z->diff_attn != 1) return fail(LK_ERR_INVALID_ARG, "diff_attn must be 0 or 1");
        if (!(z->skip_tau >= 0.f) || !std::isfinite(z->skip_tau))
            return fail(LK_ERR_INVALID_ARG, "skip_tau must be finite and >= 0");
        if (z->refresh_every < 0) return fail(LK_ERR_INVALID_ARG, "refresh_every must be >= 0");
    }
    return LK_OK;
}

// One Transformer layer ---------------------------------------------------------
struct LayerIO {
    float* x;                // residual stream [M, d]
    int M;                   // rows
    int rows_per_seq;        // rows per sequence (1 for decode)
    const int32_t* pos;      // positions (nullptr: pos_offset + row index within the sequence)
    int pos_offset;
    const u16* add;          // loop embedding added before the layer (nullptr: none)
    const int32_t* dpos;     // decode: device position t (replaces pos_offset)
    // Decode with folded norms (fold == true): x already holds `add`, and xn / ps hold
    // bf16(x * attn gain) and nparts row sums of x^2 from the producer of x.  The
    // layer's down projection leaves the same for the next layer (next_gain, after
    // adding next_add), or nothing when next_gain is null.
    bool fold;
    int nparts;
    const u16* next_gain;
    const u16* next_add;
    // Input re-injection (decode): inj = rows added to x before this layer (row-major
    // float32, added before `add`); with folded norms next_inj is added by this layer's
    // down projection before next_add, and save_x receives x before those adds.
    const float* inj;
    const float* next_inj;
    float* save_x;
    // decode-time loop skipping, folded decode: *live == 0 (no sequence left in the
    // loops) lets the layer's launches return at once (the new token's K/V write stays)
    const int32_t* live;
};

enum AttnKind { ATTN_PREFILL_DENSE, ATTN_ROWS_DENSE, ATTN_ROWS_SPARSE };

struct AttnPlan {
    AttnKind kind;
    KVLayer read;        // where attention reads K/V
    int k_loop;              // reconstruction loop for lazy reads
    const int32_t* cols;     // sparse column sets of the layer
    int n_cols, window;
    int B, T;                // prefill: batch and tokens per sequence
    int pos;                 // decode: capacity - 1 (splits are sized for the full store)
    const int32_t* dpos;     // decode: device position t
    float* mass;             // lazy loop 1: column mass output
    KVLayer scache;          // decode, loops >= 2: float16 reconstruction of the stable columns
    KVLayer ring;            // decode, loops >= 2: float16 window ring
    KVLayer full;            // prefill, loops >= 2: float16 loop-k K/V of every prompt position
                             // (full.base[0] == nullptr: the split row kernels instead)
    // difference-corrected sparse attention of a shared layer (nullptr: off).  Decode:
    // d32 [B][H hd] is set to the dense output minus the sparse one at loop 1 (cols,
    // n_cols and window given) and added at loops >= 2.  Prefill loops >= 2: d16
    // [B][T][H hd] is added, row by position.
    float* d32;
    u16* d16;
};

// End the capture running on `st` and append what it recorded (if anything) as a
// graph segment of the step being built.
int cut_segment(lk_handle* h, hipStream_t st) {
    hipGraph_t graph = nullptr;
    LK_HIP(hipStreamEndCapture(st, &graph));
    size_t n = 0;
    hipError_t e = hipGraphGetNodes(graph, nullptr, &n);
    DecodeGraph::Seg seg;
    if (e == hipSuccess && n > 0) e = hipGraphInstantiate(&seg.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(LK_ERR_HIP, std::string("decode graph: ") + hipGetErrorString(e));
    if (seg.exec) h->building->segs.push_back(std::move(seg));
    return LK_OK;
}

// Launch `fn` bracketed by timer events when its class is the instrumented one.
// While a decode step is being captured, such a launch becomes a direct segment
// of the step instead (`fn` captures its arguments by value).
template <typename F>
int timed(lk_handle* h, int cls, hipStream_t st, F fn) {
    const bool on = h->timer.wants(cls);
    if (on && h->building) {
        LK_TRY(cut_segment(h, st));
        DecodeGraph::Seg seg;
        seg.direct = fn;
        seg.cls = cls;
        h->building->segs.push_back(std::move(seg));
        LK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
        return LK_OK;
    }
    if (on) LK_HIP(h->timer.begin(st, cls));
    LK_HIP(fn());
    if (on) LK_HIP(h->timer.mark(st));
    return LK_OK;
}

int run_layer(lk_handle* h, int li, const LayerIO& io, const lk::KVWrite& kvw, const AttnPlan& ap,
              const WS& w, hipStream_t st) {
    const lk_model_cfg& c = h->c;
    // a decode step carries the device position; a prefill loop may also hand over one
    // row per sequence (one kept token), so the row count does not tell them apart
    const bool decode = io.dpos != nullptr;
    const int gcls = decode ? TC_GEMM_DECODE : TC_GEMM_PREFILL;
    const lk_layer_weights& W = h->L[li];
    const int d = c.d_model, H = c.n_heads, hd = c.head_dim, Hhd = H * hd;
    // decode-sized row counts fold the RMSNorm into the skinny GEMMs
    const bool fused_norm = io.M <= 16;
    const lk_handle::Packed PW = io.fold ? h->PL[li] : lk_handle::Packed{};
    if (io.inj) LK_HIP(lk::add_f32(io.x, io.inj, (long long)io.M * d, st));
    if (io.fold) {
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_fold_norm(w.xn, w.ps, io.nparts, c.rms_eps, PW.wqkv, io.M, h->qkv_w(), d,
                                      lk::EPI_STORE, w.qkv, nullptr, st, io.live);
        }));
    } else if (fused_norm) {
        if (io.add) LK_HIP(lk::add_rows(io.x, io.add, io.M, d, st));
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_rmsnorm(io.x, (const u16*)W.attn_norm, c.rms_eps, (const u16*)W.wqkv, io.M, h->qkv_w(),
                                    d, lk::EPI_STORE, w.qkv, nullptr, st);
        }));
    } else {
        LK_HIP(lk::rmsnorm(io.x, io.add, (const u16*)W.attn_norm, c.rms_eps, io.M, d, w.xn, nullptr, st));
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm(w.xn, (const u16*)W.wqkv, io.M, h->qkv_w(), d, lk::EPI_STORE, w.qkv, nullptr, st);
        }));
    }
    // RoPE positions: explicit, or the row index within the sequence (+ offset for decode)
    const int32_t* pos = io.pos;
    lk::KVWrite kw = kvw;
    kw.dpos = io.dpos;
    if (decode && !io.pos && io.rows_per_seq == 1) kw.rope_cs = w.rope;  // decode: one position
    if (!decode && w.rope_tab) {  // prefill: the table of every prompt position
        kw.rope_tab = w.rope_tab;
        kw.rope_rows = w.rope_rows;
    }
    // decode, loops >= 2: the sparse attention launch rotates q and writes the new
    // token's K/V itself.  (The dense launches could too, and the step time would be
    // the same: their writing workgroup gets longer by about what the separate launch
    // costs, so they keep the separate launch and measure the attention alone.)
    const bool fuse_kv = kw.rope_cs && ap.kind == ATTN_ROWS_SPARSE;
    // decode over an int8 base: the float16 MFMA kernel takes q as float16 (one rounding)
    const int q_half = decode && ap.kind == ATTN_ROWS_DENSE && ap.read.lazy && ap.read.base_bits == 8;
    if (!fuse_kv)
        LK_HIP(lk::rope_kv_write(w.qkv, io.M, io.rows_per_seq, pos, io.pos_offset, H, c.n_kv_heads, hd,
                                 h->inv_freq, w.q, kw, st, q_half));
    if (ap.kind == ATTN_PREFILL_DENSE) {
        LK_TRY(timed(h, TC_ATTN_PREFILL, st,
                     [=] { return lk::attn_prefill(w.q, ap.read, ap.B, ap.T, H, w.att, w.lse, st); }));
        if (ap.mass)
            LK_TRY(timed(h, TC_COLUMN_MASS, st,
                         [=] { return lk::column_mass(w.q, ap.read, w.lse, ap.B, ap.T, H, ap.mass, st); }));
    } else {
        lk::RowsAttn a{};
        a.q = w.q;
        a.q_half = q_half;
        a.qkv = w.qkv;
        a.rope_cs = w.rope;
        a.kvw = kw;
        a.fuse_kv = fuse_kv;
        a.qpos = io.pos;
        a.pos = ap.pos;
        a.dpos = ap.dpos;
        a.B = io.M / io.rows_per_seq;
        a.n_rows = io.rows_per_seq;
        a.H = H;
        a.kv = ap.read;
        a.k_loop = ap.k_loop;
        long long ncol_max;
        if (ap.kind == ATTN_ROWS_SPARSE) {
            a.cols = ap.cols;
            a.n_cols = ap.n_cols;
            a.window = ap.window;
            const long long limit = ap.T > 0 ? ap.T : (long long)ap.pos + 1;
            ncol_max = std::min((long long)ap.n_cols + ap.window, limit);
        } else {
            a.cols = nullptr;
            ncol_max = (long long)ap.pos + 1;
        }
        a.part = w.part;
        a.out = w.att;
        if (ap.kind == ATTN_ROWS_SPARSE && decode) {
            // decode, loops >= 2: the stable columns come from the float16 cache filled at
            // the end of prefill, the window from the float16 ring that prefill filled and
            // each decode step extends (rope_kv_write).  One launch runs over both
            // segments and the combine merges their splits.
            lk::RowsAttn d = a;
            d.kv = ap.scache;
            d.kv2 = ap.ring;
            d.chunk = kSegChunk;
            d.seg_split = ap.scache.Tmax / kSegChunk;
            d.n_splits = d.seg_split + ap.ring.Tmax / kSegChunk;
            // the launch writes the new token's K/V in a split of its own per (b, g)
            if (fuse_kv) d.nk_split = d.n_splits++;
            if ((long long)a.B * H * d.n_splits * (hd + 2) > w.part_floats)
                return fail(LK_ERR_CAPACITY, "workspace too small for attention partials");
            if (ap.d32) {
                d.diff_mode = lk::DIFF_ADD32;
                d.d32 = ap.d32;
            }
            d.live = io.live;
            LK_TRY(timed(h, TC_ATTN_DECODE_SPARSE, st, [=] { return lk::attn_rows_main(d, st); }));
            LK_HIP(lk::attn_rows_combine(d, st, io.fold));
        } else if (ap.kind == ATTN_ROWS_SPARSE && !decode && ap.full.base[0]) {
            // token-sparse prefill rows: the loop-k reconstruction is final for the stable
            // columns (cached for decode too) and for every prompt position (workspace)
            lk::RowsAttn gr{};
            gr.B = a.B;
            gr.kv = ap.read;
            gr.k_loop = ap.k_loop;
            gr.cols = ap.cols;
            gr.n_cols = ap.n_cols;
            gr.pos = ap.T - 1;
            LK_HIP(lk::gather_recon(gr, lk::GATHER_ALL_S, ap.scache.Tmax, (u16*)ap.scache.base[0],
                                    (u16*)ap.scache.base[1], st));
            LK_HIP(lk::gather_recon(gr, lk::GATHER_RING, ap.full.Tmax, (u16*)ap.full.base[0], (u16*)ap.full.base[1],
                                    st));
            if (ap.d16) {
                a.diff_mode = lk::DIFF_ADD16;
                a.d16 = ap.d16;
                a.d_rows = ap.T;
            }
            LK_TRY(timed(h, TC_ATTN_PREFILL_SPARSE, st,
                         [=] { return lk::attn_rows_prefill(a, ap.scache, ap.full, st); }));
        } else {
            if (ap.kind == ATTN_ROWS_SPARSE && ap.d16) {
                a.diff_mode = lk::DIFF_ADD16;
                a.d16 = ap.d16;
                a.d_rows = ap.T;
            }
            if (ap.kind == ATTN_ROWS_DENSE && ap.d32) {
                a.diff_mode = lk::DIFF_SET32;
                a.d32 = ap.d32;
            }
            int chunk = kRowChunk;
            if (ap.kind == ATTN_ROWS_DENSE) chunk = decode_dense_chunk(a.B * c.n_kv_heads, ncol_max);
            while ((ncol_max + chunk - 1) / chunk > kMaxSplits) chunk *= 2;
            a.chunk = chunk;
            a.n_splits = (int)((ncol_max + chunk - 1) / chunk);
            if ((long long)a.B * a.n_rows * H * a.n_splits * (hd + 2) > w.part_floats)
                return fail(LK_ERR_CAPACITY, "workspace too small for attention partials");
            const int acls = !decode ? TC_ATTN_PREFILL_SPARSE
                             : (ap.kind == ATTN_ROWS_SPARSE ? TC_ATTN_DECODE_SPARSE : TC_ATTN_DECODE_DENSE);
            LK_TRY(timed(h, acls, st, [=] { return lk::attn_rows_main(a, st); }));
            LK_HIP(lk::attn_rows_combine(a, st, io.fold));
            if (ap.kind == ATTN_ROWS_DENSE && ap.d32) {
                // the token's loop-1 sparse term, over the float16 loop-1 caches of the
                // stable columns and the window (as the later loops read theirs), taken
                // off the dense output just stored in d32
                lk::RowsAttn sp = a;
                sp.cols = ap.cols;
                sp.n_cols = ap.n_cols;
                sp.window = ap.window;
                sp.kv = ap.scache;
                sp.kv2 = ap.ring;
                sp.chunk = kSegChunk;
                sp.seg_split = ap.scache.Tmax / kSegChunk;
                sp.n_splits = sp.seg_split + ap.ring.Tmax / kSegChunk;
                sp.fuse_kv = 0;
                sp.diff_mode = lk::DIFF_SUB32;
                if (!sp.cols || !ap.scache.base[0] || !ap.ring.base[0] ||
                    (long long)a.B * H * sp.n_splits * (hd + 2) > w.part_floats)
                    return fail(LK_ERR_CAPACITY, "workspace too small for attention partials");
                LK_HIP(lk::attn_rows_main(sp, st));
                LK_HIP(lk::attn_rows_combine(sp, st, false));
            }
        }
    }
    const int act = c.ffn_act == LK_ACT_SWIGLU ? lk::EPI_SWIGLU : lk::EPI_GELU;
    if (io.fold) {
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_fold_add(w.att, PW.wo, io.M, d, Hhd, io.x, nullptr, (const u16*)W.ffn_norm, w.xn, w.ps,
                                     st, nullptr, nullptr, io.live);
        }));
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_fold_norm(w.xn, w.ps, d / 8, c.rms_eps, PW.w_in, io.M, c.ffn_dim, d, act, nullptr,
                                      w.act, st, io.live);
        }));
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_fold_add(w.act, PW.w_down, io.M, d, c.ffn_dim, io.x, io.next_add, io.next_gain, w.xn,
                                     w.ps, st, io.next_inj, io.save_x, io.live);
        }));
        return LK_OK;
    }
    LK_TRY(timed(h, gcls, st,
                 [=] { return lk::gemm(w.att, (const u16*)W.wo, io.M, d, Hhd, lk::EPI_ADD, io.x, nullptr, st); }));
    if (fused_norm) {
        LK_TRY(timed(h, gcls, st, [=] {
            return lk::gemm_rmsnorm(io.x, (const u16*)W.ffn_norm, c.rms_eps, (const u16*)W.w_in, io.M, c.ffn_dim, d,
                                    act, nullptr, w.act, st);
        }));
    } else {
        LK_HIP(lk::rmsnorm(io.x, nullptr, (const u16*)W.ffn_norm, c.rms_eps, io.M, d, w.xn, nullptr, st));
        LK_TRY(timed(h, gcls, st,
                     [=] { return lk::gemm(w.xn, (const u16*)W.w_in, io.M, c.ffn_dim, d, act, nullptr, w.act, st); }));
    }
    LK_TRY(timed(h, gcls, st, [=] {
        return lk::gemm(w.act, (const u16*)W.w_down, io.M, d, c.ffn_dim, lk::EPI_ADD, io.x, nullptr, st);
    }));
    return LK_OK;
}

// Difference-corrected attention at prefill loop 1 of shared layer r: the sparse term
// of every prompt row (its column set over the loop-1 reconstruction), taken off the
// dense output the layer left in w.att, into the float16 rows of layer r in w.dprompt.
// Runs after the layer picked its column sets; w.q still holds the rotated queries.
int diff_prompt_rows(lk_handle* h, lk_kv_store* s, int r, const WS& w, int B, int T, hipStream_t st) {
    const lk_model_cfg& c = h->c;
    const long long Hhd = (long long)c.n_heads * c.head_dim;
    lk::RowsAttn a{};
    a.q = w.q;
    a.qpos = w.sel;
    a.B = B;
    a.n_rows = T;
    a.H = c.n_heads;
    a.kv = lazy_layer(s, r);
    a.k_loop = 1;
    a.cols = col_sets(s, r);
    a.n_cols = s->lay.n_cols;
    a.window = h->z.window;
    a.out = w.att;
    a.part = w.part;
    a.diff_mode = lk::DIFF_OUT16;
    a.d16 = w.dprompt + (long long)r * B * T * Hhd;
    a.d_rows = T;
    LK_HIP(lk::iota_rows(w.sel, B, T, st));
    if (w.fr_cap) {
        // the loop-1 stable-column cache of layer r (filled again for decode once the
        // loops are done)
        const KVLayer sc = scache_layer(s, 1, r);
        KVLayer fr = sc;
        fr.Tmax = w.fr_cap;
        fr.base[0] = w.frk;
        fr.base[1] = w.frv;
        lk::RowsAttn gr{};
        gr.B = B;
        gr.kv = a.kv;
        gr.k_loop = 1;
        gr.cols = a.cols;
        gr.n_cols = a.n_cols;
        gr.pos = T - 1;
        LK_HIP(lk::gather_recon(gr, lk::GATHER_ALL_S, sc.Tmax, (u16*)sc.base[0], (u16*)sc.base[1], st));
        LK_HIP(lk::gather_recon(gr, lk::GATHER_RING, fr.Tmax, w.frk, w.frv, st));
        LK_HIP(lk::attn_rows_prefill(a, sc, fr, st));
        return LK_OK;
    }
    const long long ncol = std::min((long long)a.n_cols + a.window, (long long)T);
    a.chunk = kRowChunk;
    a.n_splits = (int)((ncol + kRowChunk - 1) / kRowChunk);
    if ((long long)B * T * c.n_heads * a.n_splits * (c.head_dim + 2) > w.part_floats)
        return fail(LK_ERR_CAPACITY, "workspace too small for attention partials");
    LK_HIP(lk::attn_rows_main(a, st));
    LK_HIP(lk::attn_rows_combine(a, st, false));
    return LK_OK;
}

lk::KVWrite plain_write(const KVLayer& L) {
    lk::KVWrite k{};
    k.kind = 0;
    k.layer = L;
    return k;
}

// Fill the float16 decode caches of loops ck0..K from the base and residuals: the
// stable-column reconstructions (when with_s; always for loop 1, which prefill does
// not cache as it goes) and the window rings ending at position `last` (the rows of
// positions up to `last` that decode can read).
int fill_decode_caches(lk_kv_store* s, bool with_s, int last, hipStream_t st) {
    if (s->K < 2) return LK_OK;
    for (int k = s->lay.ck0; k <= s->K; ++k)
        for (int r = 0; r < s->h->c.n_shared; ++r) {
            lk::RowsAttn g{};
            g.B = s->B;
            g.kv = lazy_layer(s, r);
            g.k_loop = k;
            g.cols = col_sets(s, r);
            g.n_cols = s->lay.n_cols;
            g.pos = last;
            if (with_s || k == 1) {
                const KVLayer L = scache_layer(s, k, r);
                LK_HIP(lk::gather_recon(g, lk::GATHER_ALL_S, s->lay.ncs, (u16*)L.base[0], (u16*)L.base[1], st));
            }
            const KVLayer Rg = scache_layer(s, k, r, true);
            LK_HIP(lk::gather_recon(g, lk::GATHER_RING, s->lay.wr, (u16*)Rg.base[0], (u16*)Rg.base[1], st));
        }
    return LK_OK;
}

bool same_cfg(const lk_model_cfg& a, const lk_model_cfg& b) {
    return a.vocab == b.vocab && a.d_model == b.d_model && a.n_heads == b.n_heads && a.n_kv_heads == b.n_kv_heads &&
           a.head_dim == b.head_dim && a.ffn_dim == b.ffn_dim && a.ffn_act == b.ffn_act &&
           a.n_prelude == b.n_prelude && a.n_shared == b.n_shared && a.n_loops == b.n_loops &&
           a.n_coda == b.n_coda && a.rms_eps == b.rms_eps && a.rope_theta == b.rope_theta &&
           a.input_reinject == b.input_reinject;
}

bool same_lazy(const lk_lazy_cfg& a, const lk_lazy_cfg& b) {
    return a.mode == b.mode && a.rho == b.rho && a.top_s == b.top_s && a.window == b.window &&
           a.base_bits == b.base_bits && a.res_bits == b.res_bits && a.group == b.group &&
           a.stale_keys == b.stale_keys && a.refresh_every == b.refresh_every && a.diff_attn == b.diff_attn &&
           a.skip_tau == b.skip_tau;
}

}  // namespace

// =============================================================================
extern "C" {

const char* lk_last_error(void) { return g_err.c_str(); }

int lk_create(const lk_model_cfg* cfg, const lk_lazy_cfg* lazy, const lk_weights* w, lk_handle** out) {
    if (!out) return fail(LK_ERR_INVALID_ARG, "null out");
    *out = nullptr;
    LK_TRY(check_cfg(cfg, lazy));
    if (!w || !w->tok_emb || !w->loop_emb || !w->final_norm || !w->layers)
        return fail(LK_ERR_INVALID_ARG, "null weight pointer");
    const int L = cfg->n_prelude + cfg->n_shared + cfg->n_coda;
    for (int i = 0; i < L; ++i) {
        const lk_layer_weights& l = w->layers[i];
        if (!l.attn_norm || !l.wqkv || !l.wo || !l.ffn_norm || !l.w_in || !l.w_down)
            return fail(LK_ERR_INVALID_ARG, "null layer weight pointer in layer " + std::to_string(i));
    }
    lk_handle* h = new lk_handle();
    h->c = *cfg;
    h->z = *lazy;
    h->tok = (const u16*)w->tok_emb;
    h->lemb = (const u16*)w->loop_emb;
    h->fnorm = (const u16*)w->final_norm;
    h->L.assign(w->layers, w->layers + L);
    for (int i = 0; i < cfg->head_dim / 2; ++i)
        h->inv_freq[i] = std::pow((double)cfg->rope_theta, -2.0 * i / (double)cfg->head_dim);
    *out = h;
    return LK_OK;
}

void lk_destroy(lk_handle* h) { delete h; }

int lk_effective_depth(const lk_handle* h, int32_t* depth) {
    if (!h || !depth) return fail(LK_ERR_INVALID_ARG, "null argument");
    *depth = h->c.n_prelude + h->c.n_shared * h->c.n_loops + h->c.n_coda;
    return LK_OK;
}

int lk_kv_store_alloc(lk_handle* h, int32_t batch, int32_t prompt_tokens, int32_t max_tokens, void* dev_buf,
                      size_t buf_bytes, void* stream, lk_kv_store** out, size_t* need_bytes) {
    if (!h || !need_bytes) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (batch < 1 || prompt_tokens < 1 || max_tokens < prompt_tokens)
        return fail(LK_ERR_INVALID_ARG, "need batch >= 1 and 1 <= prompt_tokens <= max_tokens");
    const StoreLayout lay = store_layout(h, batch, prompt_tokens, max_tokens);
    *need_bytes = lay.total;
    if (!dev_buf) return LK_OK;
    if (!out) return fail(LK_ERR_INVALID_ARG, "null out");
    if (buf_bytes < lay.total) return fail(LK_ERR_CAPACITY, "store buffer too small");
    if ((uintptr_t)dev_buf % kAlign) return fail(LK_ERR_INVALID_ARG, "store buffer must be 256-byte aligned");
    lk_kv_store* s = new lk_kv_store();
    s->h = h;
    s->B = batch;
    s->Tp = prompt_tokens;
    s->Tmax = max_tokens;
    s->Tpad = pad8(max_tokens);
    s->t = 0;
    s->K = h->c.n_loops;
    s->prefilled = false;
    s->lay = lay;
    s->buf = (char*)dev_buf;
    s->f_tok = s->f_cols = nullptr;
    s->keep_codes = 0;
    if (h->lazy()) {
        hipError_t e = lk::fill_i32((int32_t*)range_flag(s), 0, 1, (hipStream_t)stream);
        if (e == hipSuccess)
            e = lk::fill_i32(slot_map(s, 2), -1, (long long)(h->c.n_loops - 1) * batch * s->Tpad, (hipStream_t)stream);
        if (e != hipSuccess) {
            delete s;
            return fail(LK_ERR_HIP, std::string("store clear: ") + hipGetErrorString(e));
        }
    }
    *out = s;
    return LK_OK;
}

void lk_kv_store_release(lk_kv_store* s) {
    if (!s) return;
    if (s->h && s->h->graph.store == s) {  // its captured decode step refers to this store
        (void)hipDeviceSynchronize();
        s->h->graph.reset();
    }
    delete s;
}

int lk_kv_store_bytes_used(const lk_kv_store* s, size_t* shared, size_t* total) {
    if (!s || !shared || !total) return fail(LK_ERR_INVALID_ARG, "null argument");
    store_bytes(s, shared, total);
    return LK_OK;
}

int lk_kv_store_cache_bytes(const lk_kv_store* s, size_t* bytes) {
    if (!s || !bytes) return fail(LK_ERR_INVALID_ARG, "null argument");
    *bytes = s->lay.scache_bytes;
    return LK_OK;
}

int lk_kv_store_set_loops(lk_kv_store* s, int32_t n_loops) {
    if (!s) return fail(LK_ERR_INVALID_ARG, "null store");
    if (s->prefilled || s->t > 0) return fail(LK_ERR_STATE, "the loop count is set before prefill");
    if (n_loops < 1 || n_loops > s->h->c.n_loops) return fail(LK_ERR_INVALID_ARG, "n_loops outside [1, model n_loops]");
    s->K = n_loops;
    return LK_OK;
}

int lk_kv_store_length(const lk_kv_store* s, int32_t* tokens) {
    if (!s || !tokens) return fail(LK_ERR_INVALID_ARG, "null argument");
    *tokens = s->t;
    return LK_OK;
}

int lk_kv_store_range_check(lk_kv_store* s, int32_t clear, int32_t* out_of_range, void* stream) {
    if (!s || !out_of_range) return fail(LK_ERR_INVALID_ARG, "null argument");
    *out_of_range = 0;
    if (!s->h->lazy()) return LK_OK;  // bf16 rows only: the flag is never raised
    hipStream_t st = (hipStream_t)stream;
    uint32_t flag = 0;
    LK_HIP(hipMemcpyAsync(&flag, range_flag(s), sizeof(flag), hipMemcpyDeviceToHost, st));
    LK_HIP(hipStreamSynchronize(st));
    *out_of_range = flag != 0;
    if (clear) LK_HIP(lk::fill_i32((int32_t*)range_flag(s), 0, 1, st));
    return LK_OK;
}

int lk_kv_store_view(const lk_kv_store* s, lk_store_view* v) {
    if (!s || !v) return fail(LK_ERR_INVALID_ARG, "null argument");
    std::memset(v, 0, sizeof(*v));
    const lk_handle* h = s->h;
    v->row_stride = s->Tpad;
    if (h->c.n_prelude + h->c.n_coda > 0) v->dense = s->buf + s->lay.dense;
    if (h->z.mode != LK_MODE_LAZY) {
        v->loop_rows = s->buf + s->lay.loop_rows;
        return LK_OK;
    }
    v->base_codes = s->buf + s->lay.base;
    v->base_scales = h->z.base_bits == 16 ? nullptr : s->buf + s->lay.base_sc;
    v->res_codes = s->buf + s->lay.res;
    v->res_scales = h->z.res_bits == 16 ? nullptr : s->buf + s->lay.res_sc;
    v->slot_maps = (int32_t*)(s->buf + s->lay.slot);
    v->columns = (int32_t*)(s->buf + s->lay.cols);
    v->slots = s->lay.slots;
    v->n_selected = s->lay.n_sel;
    v->n_columns = s->lay.n_cols;
    v->res_row_bytes = s->lay.res_row_b;
    if (s->lay.scache_bytes) {
        v->decode_cache = s->buf + s->lay.scache;
        v->cache_rows = s->lay.ncs;
        v->ring_rows = s->lay.wr;
        v->first_cached_loop = s->lay.ck0;
    }
    return LK_OK;
}

int lk_kv_store_force_selection(lk_kv_store* s, const int32_t* d_tokens, const int32_t* d_columns) {
    if (!s) return fail(LK_ERR_INVALID_ARG, "null store");
    if (!s->h->lazy()) return fail(LK_ERR_STATE, "selection exists only in lazy mode");
    s->f_tok = d_tokens;
    s->f_cols = d_columns;
    return LK_OK;
}

int lk_kv_store_export(const lk_kv_store* s, void* host_buf, size_t buf_bytes, size_t* need_bytes, void* stream) {
    if (!s || !need_bytes) return fail(LK_ERR_INVALID_ARG, "null argument");
    const size_t body = s->lay.scache;  // everything before the derived decode caches
    *need_bytes = sizeof(lk_store_snapshot) + body;
    if (!host_buf) return LK_OK;
    if (buf_bytes < *need_bytes) return fail(LK_ERR_CAPACITY, "snapshot buffer too small");
    lk_store_snapshot hd;
    std::memset(&hd, 0, sizeof(hd));
    hd.magic = LK_SNAPSHOT_MAGIC;
    hd.header_bytes = sizeof(lk_store_snapshot);
    hd.version = LK_SNAPSHOT_VERSION;
    hd.cfg = s->h->c;
    hd.lazy = s->h->z;
    hd.batch = s->B;
    hd.prompt_tokens = s->Tp;
    hd.max_tokens = s->Tmax;
    hd.loops = s->K;
    hd.tokens = s->t;
    hd.prefilled = s->prefilled ? 1 : 0;
    hd.body_bytes = body;
    std::memcpy(host_buf, &hd, sizeof(hd));
    hipStream_t st = (hipStream_t)stream;
    LK_HIP(hipMemcpyAsync((char*)host_buf + sizeof(hd), s->buf, body, hipMemcpyDeviceToHost, st));
    LK_HIP(hipStreamSynchronize(st));
    return LK_OK;
}

int lk_kv_store_import(lk_kv_store* s, const void* host_buf, size_t bytes, void* stream) {
    if (!s || !host_buf) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (bytes < sizeof(lk_store_snapshot)) return fail(LK_ERR_INVALID_ARG, "snapshot shorter than its header");
    lk_store_snapshot hd;
    std::memcpy(&hd, host_buf, sizeof(hd));
    const lk_handle* h = s->h;
    if (hd.magic != LK_SNAPSHOT_MAGIC || hd.header_bytes != sizeof(lk_store_snapshot) ||
        hd.version != LK_SNAPSHOT_VERSION)
        return fail(LK_ERR_INVALID_ARG, "not a store snapshot of this version");
    if (!same_cfg(hd.cfg, h->c) || !same_lazy(hd.lazy, h->z))
        return fail(LK_ERR_INVALID_ARG, "snapshot written under another model config or cache policy");
    if (hd.batch != s->B || hd.prompt_tokens != s->Tp || hd.max_tokens != s->Tmax)
        return fail(LK_ERR_INVALID_ARG, "snapshot of a store with another batch, prompt or capacity");
    if (hd.loops < 1 || hd.loops > h->c.n_loops) return fail(LK_ERR_INVALID_ARG, "snapshot loop count out of range");
    if (hd.prefilled ? (hd.tokens < s->Tp || hd.tokens > s->Tmax) : hd.tokens != 0)
        return fail(LK_ERR_INVALID_ARG, "snapshot length inconsistent with its prefill flag");
    if (hd.body_bytes != s->lay.scache) return fail(LK_ERR_INVALID_ARG, "snapshot body size differs from the store's");
    if (bytes - sizeof(hd) < hd.body_bytes) return fail(LK_ERR_INVALID_ARG, "snapshot truncated");
    if (h->graph.store == s) {  // its captured decode step may be in flight
        LK_HIP(hipDeviceSynchronize());
        s->h->graph.reset();
    }
    hipStream_t st = (hipStream_t)stream;
    LK_HIP(hipMemcpyAsync(s->buf, (const char*)host_buf + sizeof(hd), hd.body_bytes, hipMemcpyHostToDevice, st));
    s->t = hd.tokens;
    s->K = hd.loops;
    s->prefilled = hd.prefilled != 0;
    LK_HIP(lk::fill_i32(dev_pos(s), hd.tokens, 1, st));
    if (s->lay.scache_bytes) {
        LK_HIP(lk::fill_i32((int32_t*)(s->buf + s->lay.scache), 0, (long long)(s->lay.scache_bytes / 4), st));
        if (s->prefilled && s->K >= 2) LK_TRY(fill_decode_caches(s, true, s->t - 1, st));
    }
    LK_HIP(hipStreamSynchronize(st));
    return LK_OK;
}

int lk_kv_store_keep_codes(lk_kv_store* s, int32_t enable) {
    if (!s) return fail(LK_ERR_INVALID_ARG, "null store");
    if (!s->h->lazy()) return fail(LK_ERR_STATE, "codes exist only in lazy mode");
    s->keep_codes = enable ? 1 : 0;
    return LK_OK;
}

int lk_workspace_bytes(lk_handle* h, int32_t batch, int32_t tokens, size_t* bytes) {
    if (!h || !bytes) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (batch < 1 || tokens < 1) return fail(LK_ERR_INVALID_ARG, "batch and tokens must be >= 1");
    *bytes = ws_layout(h, batch, tokens, nullptr).total;
    return LK_OK;
}

int lk_looped_prefill(lk_handle* h, lk_kv_store* s, const int32_t* d_ids, int32_t B, int32_t T, float* d_out,
                      void* d_ws, size_t ws_bytes, void* stream) {
    if (!h || !s || !d_ids || !d_out || !d_ws) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (s->h != h) return fail(LK_ERR_INVALID_ARG, "store belongs to another handle");
    if (B != s->B || T != s->Tp) return fail(LK_ERR_INVALID_ARG, "B and T must match the store");
    const WS w = ws_layout(h, B, T, (char*)d_ws);
    if (ws_bytes < w.total) return fail(LK_ERR_CAPACITY, "workspace too small");
    if ((uintptr_t)d_ws % kAlign) return fail(LK_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const lk_model_cfg& c = h->c;
    const int P = c.n_prelude, R = c.n_shared, K = s->K, Q = c.n_coda, d = c.d_model;
    const int M = B * T;
    const bool inject = c.input_reinject != 0;
    h->timer.new_call();
    if (h->lazy())
        LK_HIP(lk::fill_i32(slot_map(s, 2), -1, (long long)(K - 1) * B * s->Tpad, st));
    s->t = 0;
    s->prefilled = false;
    if (w.rope_rows) LK_HIP(lk::rope_table(h->inv_freq, w.rope_rows, c.head_dim, w.rope_tab, st));
    LK_HIP(lk::embed(d_ids, h->tok, w.h, M, d, c.vocab, st));

    LayerIO io{w.h, M, T, nullptr, 0, nullptr};
    AttnPlan dense_plan{};
    dense_plan.kind = ATTN_PREFILL_DENSE;
    dense_plan.B = B;
    dense_plan.T = T;
    for (int li = 0; li < P; ++li) {
        dense_plan.read = dense_layer(s, li);
        LK_TRY(run_layer(h, li, io, plain_write(dense_plan.read), dense_plan, w, st));
    }
    if (!h->lazy()) {
        if (inject) LK_HIP(lk::copy_f32(w.h, w.h0, (long long)M * d, st));  // e = prelude output
        for (int k = 1; k <= K; ++k)
            for (int r = 0; r < R; ++r) {
                if (inject && k >= 2 && r == 0) LK_HIP(lk::add_f32(w.h, w.h0, (long long)M * d, st));
                io.add = (r == 0) ? h->lemb + (long long)(k - 1) * d : nullptr;
                dense_plan.read = loop_layer(s, k, r);
                LK_TRY(run_layer(h, P + r, io, plain_write(dense_plan.read), dense_plan, w, st));
            }
        io.add = nullptr;
    } else {
        const bool diff = h->z.diff_attn && K >= 2;
        LK_HIP(lk::copy_f32(w.h, w.h0, (long long)M * d, st));
        // loop 1: dense over every token; writes the base and picks the column sets
        for (int r = 0; r < R; ++r) {
            io.add = (r == 0) ? h->lemb : nullptr;
            AttnPlan ap = dense_plan;
            ap.read = lazy_layer(s, r);
            ap.mass = w.mass;
            lk::KVWrite kw{};
            kw.kind = 1;
            kw.layer = ap.read;
            kw.keep_codes = s->keep_codes;
            kw.range_flag = range_flag(s);
            LK_TRY(run_layer(h, P + r, io, kw, ap, w, st));
            int32_t* cols = col_sets(s, r);
            const int nc = s->lay.n_cols;
            if (s->f_cols) {
                LK_HIP(hipMemcpyAsync(cols, s->f_cols + (long long)r * B * c.n_kv_heads * nc,
                                      (size_t)B * c.n_kv_heads * nc * 4, hipMemcpyDeviceToDevice, st));
            } else {
                LK_HIP(lk::topk_rows(w.mass, B * c.n_kv_heads, T, nc, cols, st));
            }
            if (diff) LK_TRY(diff_prompt_rows(h, s, r, w, B, T, st));
        }
        io.add = nullptr;
        if (K >= 2) LK_HIP(lk::delta_keys(w.h, w.h0, M, d, w.keys, st));
        // decode caches: rows not written below stay zero
        if (K >= 2)
            LK_HIP(lk::fill_i32((int32_t*)(s->buf + s->lay.scache), 0, (long long)(s->lay.scache_bytes / 4), st));
        KVLayer full{};
        if (w.fr_cap) {
            full = scache_layer(s, 2, 0);  // a float16 plain layer, re-pointed at the workspace
            full.Tmax = w.fr_cap;
            full.base[0] = w.frk;
            full.base[1] = w.frv;
        }
        for (int k = 2; k <= K; ++k) {
            const int n = loop_rows(s, k);
            if (refresh_loop(h->z, k)) {  // every token
                LK_HIP(lk::iota_rows(w.sel, B, n, st));
            } else if (s->f_tok) {
                LK_HIP(hipMemcpyAsync(w.sel, s->f_tok + (long long)(k - 2) * B * n, (size_t)B * n * 4,
                                      hipMemcpyDeviceToDevice, st));
            } else {
                LK_HIP(lk::topk_rows(w.keys, B, T, n, w.sel, st));
            }
            LK_HIP(lk::gather_rows(w.h, w.sel, B, n, T, d, h->lemb + (long long)(k - 1) * d, w.xc,
                                   slot_map(s, k), s->Tpad, st, inject ? w.h0 : nullptr));
            LayerIO cio{w.xc, B * n, n, w.sel, 0, nullptr};
            for (int r = 0; r < R; ++r) {
                AttnPlan ap{};
                ap.kind = ATTN_ROWS_SPARSE;
                ap.read = lazy_layer(s, r);
                ap.k_loop = k;
                ap.cols = col_sets(s, r);
                ap.n_cols = s->lay.n_cols;
                ap.window = h->z.window;
                ap.T = T;
                ap.scache = scache_layer(s, k, r);
                ap.full = full;
                if (diff) ap.d16 = w.dprompt + (long long)r * M * c.n_heads * c.head_dim;
                lk::KVWrite kw{};
                kw.kind = 2;
                kw.layer = ap.read;
                kw.loop = k;
                kw.slot_base = 0;
                kw.keep_codes = s->keep_codes;
                kw.range_flag = range_flag(s);
                LK_TRY(run_layer(h, P + r, cio, kw, ap, w, st));
            }
            if (k < K) {
                // the next loop's keys: the change of every recomputed token; a carried
                // token's is zero, or (stale_keys) stays the one it has
                if (!h->z.stale_keys) LK_HIP(lk::fill_f32(w.keys, 0.f, (long long)M, st));
                LK_HIP(lk::scatter_rows(w.xc, w.sel, B, n, T, d, w.h, w.keys, st));
            } else {
                LK_HIP(lk::scatter_rows(w.xc, w.sel, B, n, T, d, w.h, nullptr, st));
            }
        }
        // The stable columns' and the prompt tail's loop-k reconstructions are final
        // now: cache them (float16) for decode (the stable columns already are when the
        // loop used them through the cache).
        LK_TRY(fill_decode_caches(s, !w.fr_cap, T - 1, st));
    }
    for (int j = 0; j < Q; ++j) {
        dense_plan.read = dense_layer(s, P + j);
        LK_TRY(run_layer(h, P + R + j, io, plain_write(dense_plan.read), dense_plan, w, st));
    }
    LK_HIP(lk::rmsnorm(w.h, nullptr, h->fnorm, c.rms_eps, M, d, nullptr, d_out, st));
    LK_HIP(lk::fill_i32(dev_pos(s), T, 1, st));
    s->t = T;
    s->prefilled = true;
    return LK_OK;
}

}  // extern "C"

namespace {

// Bytes of the packed decode weights (0 when the shapes do not take the folded products).
size_t packed_weight_bytes(const lk_handle* h) {
    const lk_model_cfg& c = h->c;
    const int d = c.d_model, Hhd = c.n_heads * c.head_dim, F = c.ffn_dim;
    const int fin = c.ffn_act == LK_ACT_SWIGLU ? 2 : 1;
    if (!lk::gemm_fold_supported(8, h->qkv_w(), d) || !lk::gemm_fold_supported(8, d, Hhd) ||
        !lk::gemm_fold_supported(8, F, d) || !lk::gemm_fold_supported(8, d, F))
        return 0;
    const size_t per = ((size_t)h->qkv_w() * d + (size_t)d * Hhd + (size_t)fin * F * d + (size_t)d * F) * 2;
    return per * h->L.size();
}

// Pack the layer projections into buf (at least packed_weight_bytes(h)) on st.
int pack_decode_weights(lk_handle* h, void* buf, hipStream_t st) {
    const lk_model_cfg& c = h->c;
    const int d = c.d_model, Hhd = c.n_heads * c.head_dim, F = c.ffn_dim;
    const int fin = c.ffn_act == LK_ACT_SWIGLU ? 2 : 1;
    u16* p = (u16*)buf;
    h->PL.resize(h->L.size());
    for (size_t i = 0; i < h->L.size(); ++i) {
        const lk_layer_weights& W = h->L[i];
        lk_handle::Packed& P = h->PL[i];
        auto pack = [&](const void* src, long long rows, int K, const u16** dst) {
            hipError_t e = lk::pack_weights((const u16*)src, rows, K, p, st);
            *dst = p;
            p += (size_t)rows * K;
            return e;
        };
        LK_HIP(pack(W.wqkv, h->qkv_w(), d, &P.wqkv));
        LK_HIP(pack(W.wo, d, Hhd, &P.wo));
        LK_HIP(pack(W.w_in, (long long)fin * F, d, &P.w_in));
        LK_HIP(pack(W.w_down, d, F, &P.w_down));
    }
    h->pk_buf = buf;
    return LK_OK;
}

// Enqueue one decode step: ids from w.ids, output rows to w.out, position from the
// store's device counter (incremented at the end).  Nothing here depends on the
// host's copy of the position, so the same launches serve every step.
int enqueue_decode(lk_handle* h, lk_kv_store* s, const WS& w, hipStream_t st) {
    const lk_model_cfg& c = h->c;
    const int P = c.n_prelude, R = c.n_shared, K = s->K, Q = c.n_coda, d = c.d_model;
    const int B = s->B;
    const bool inject = c.input_reinject != 0;
    const int32_t* dpos = dev_pos(s);
    const bool skip = h->lazy() && h->z.skip_tau > 0.f && K >= 2;
    h->timer.new_call();
    // The layer applications of one step, in order.
    struct App {
        int li;
        const u16* add;
        lk::KVWrite kw;
        AttnPlan ap;
        bool inj;  // re-injection before this layer (first shared layer of loops >= 2)
    };
    std::vector<App> apps;
    apps.reserve((size_t)P + (size_t)R * K + Q);
    AttnPlan dense{};
    dense.kind = ATTN_ROWS_DENSE;
    dense.k_loop = 1;
    dense.pos = s->Tmax - 1;  // splits are sized for the store's capacity
    dense.dpos = dpos;
    for (int li = 0; li < P; ++li) {
        dense.read = dense_layer(s, li);
        apps.push_back({li, nullptr, plain_write(dense.read), dense, false});
    }
    for (int k = 1; k <= K; ++k) {
        for (int r = 0; r < R; ++r) {
            const u16* add = (r == 0) ? h->lemb + (long long)(k - 1) * d : nullptr;
            const bool inj = inject && k >= 2 && r == 0;
            if (!h->lazy()) {
                dense.read = loop_layer(s, k, r);
                apps.push_back({P + r, add, plain_write(dense.read), dense, inj});
                continue;
            }
            AttnPlan ap{};
            ap.read = lazy_layer(s, r);
            ap.pos = s->Tmax - 1;
            ap.dpos = dpos;
            lk::KVWrite kw{};
            kw.layer = ap.read;
            kw.keep_codes = s->keep_codes;
            kw.range_flag = range_flag(s);
            if (skip) kw.active = w.sk_act;
            kw.tok_recon = w.tokrec + (long long)r * B * 2 * c.n_kv_heads * c.head_dim;
            if (h->z.diff_attn && K >= 2) {
                ap.d32 = w.dstep + (long long)r * B * c.n_heads * c.head_dim;
                ap.cols = col_sets(s, r);
                ap.n_cols = s->lay.n_cols;
                ap.window = h->z.window;
                if (k == 1) {  // the loop-1 sparse term reads the loop-1 caches
                    ap.scache = scache_layer(s, 1, r);
                    ap.ring = scache_layer(s, 1, r, true);
                    kw.ring = ap.ring;
                    kw.ring_on = 1;
                }
            }
            if (k == 1) {
                ap.kind = ATTN_ROWS_DENSE;
                ap.k_loop = 1;
                kw.kind = 1;
            } else {
                ap.kind = ATTN_ROWS_SPARSE;
                ap.k_loop = k;
                ap.cols = col_sets(s, r);
                ap.n_cols = s->lay.n_cols;
                ap.window = h->z.window;
                ap.scache = scache_layer(s, k, r);
                ap.ring = scache_layer(s, k, r, true);
                kw.ring = ap.ring;
                kw.ring_on = 1;
                kw.kind = 2;
                kw.loop = k;
                kw.slot_base = (long long)loop_rows(s, k) - s->Tp;  // slot = n_k + (t - T)
                kw.slot_map_k = slot_map(s, k);
            }
            apps.push_back({P + r, add, kw, ap, inj});
        }
    }
    for (int j = 0; j < Q; ++j) {
        dense.read = dense_layer(s, P + j);
        apps.push_back({P + R + j, nullptr, plain_write(dense.read), dense, false});
    }
    // Folded norms: every projection input is prepared by the kernel that produced x.
    const bool fold = B <= 8 && h->pk_buf != nullptr;
    LK_HIP(lk::embed(w.ids, h->tok, w.h, B, d, c.vocab, st));
    LK_HIP(lk::rope_angles(dpos, h->inv_freq, c.head_dim, w.rope, st));
    if (skip) {  // every token enters the loops; h_0 is the prelude output
        LK_HIP(lk::fill_i32(w.sk_act, 1, B, st));
        LK_HIP(lk::fill_i32(w.sk_live, B, 1, st));
        if (P == 0) LK_HIP(lk::copy_f32(w.h, w.sk_prev, (long long)B * d, st));
    }
    // re-injection: e = the prelude output (the embedding when there is no prelude)
    if (inject && K >= 2 && P == 0) LK_HIP(lk::copy_f32(w.h, w.h0, (long long)B * d, st));
    if (fold)
        LK_HIP(lk::norm_prep(w.h, apps[0].add, (const u16*)h->L[apps[0].li].attn_norm, B, d, w.xn, w.ps, st));
    int nparts_next = 0;  // the next layer's normed input was prepared by norm_prep
    for (size_t i = 0; i < apps.size(); ++i) {
        const App& a = apps[i];
        LayerIO io{w.h, B, 1, nullptr, 0, fold ? nullptr : a.add, dpos};
        io.fold = fold;
        io.nparts = i == 0 || nparts_next ? 1 : d / 8;
        nparts_next = 0;
        // position of a shared-layer application in the loops
        const long long li_loop = (long long)i - P;
        const int kk = li_loop >= 0 && li_loop < (long long)K * R ? (int)(li_loop / R) + 1 : 0;
        const int rr = kk ? (int)(li_loop % R) : -1;
        if (i + 1 < apps.size()) {
            io.next_gain = (const u16*)h->L[apps[i + 1].li].attn_norm;
            io.next_add = apps[i + 1].add;
            if (fold && apps[i + 1].inj) io.next_inj = w.h0;
        }
        if (inject && K >= 2 && P > 0) {
            if (fold && i + 1 == (size_t)P) io.save_x = w.h0;  // x after the last prelude layer
            if (!fold && i == (size_t)P) LK_HIP(lk::copy_f32(w.h, w.h0, (long long)B * d, st));
        }
        if (!fold && a.inj) io.inj = w.h0;
        bool copy_e = false;  // skipping: h_0 = the prelude output, saved by the layer
        if (skip && P > 0) {
            if (fold && i + 1 == (size_t)P) {
                if (io.save_x) copy_e = true;
                else io.save_x = w.sk_prev;
            }
            if (!fold && i == (size_t)P) LK_HIP(lk::copy_f32(w.h, w.sk_prev, (long long)B * d, st));
        }
        if (skip && kk >= 2 && rr == 0)  // h_{k-1}: saved by the last layer (folded) or in h
            LK_HIP(lk::skip_gate(fold ? w.sk_save : w.h, w.sk_prev, w.sk_act, w.sk_live, h->z.skip_tau, B, d, st));
        // folded decode: the launches of loops >= 2 return at once when no sequence is left
        if (skip && fold && kk >= 2) io.live = w.sk_live;
        if (skip && fold && kk >= 1 && kk < K && rr == R - 1) io.save_x = w.sk_save;
        LK_TRY(run_layer(h, a.li, io, a.kw, a.ap, w, st));
        if (copy_e) LK_HIP(lk::copy_f32(io.save_x, w.sk_prev, (long long)B * d, st));
        if (skip && kk == K && rr == R - 1) {
            LK_HIP(lk::skip_restore(w.h, w.sk_prev, w.sk_act, B, d, st));
            if (fold && i + 1 < apps.size()) {  // the coda's first normed input, again
                LK_HIP(lk::norm_prep(w.h, nullptr, (const u16*)h->L[apps[i + 1].li].attn_norm, B, d, w.xn, w.ps,
                                     st));
                nparts_next = 1;
            }
        }
    }
    LK_HIP(lk::rmsnorm(w.h, nullptr, h->fnorm, c.rms_eps, B, d, nullptr, w.out, st));
    LK_HIP(lk::add_i32(dev_pos(s), 1, st));
    return LK_OK;
}

// Capture one decode step on `st` into h->graph (segments as described there).
int capture_decode(lk_handle* h, lk_kv_store* s, const WS& w, hipStream_t st) {
    LK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
    h->building = &h->graph;
    int rc = enqueue_decode(h, s, w, st);
    if (rc == LK_OK) rc = cut_segment(h, st);
    h->building = nullptr;
    if (rc != LK_OK) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone) {
            hipGraph_t g = nullptr;
            (void)hipStreamEndCapture(st, &g);
            if (g) (void)hipGraphDestroy(g);
        }
        h->graph.reset();
    }
    return rc;
}

// Decode workspace for callers that cannot allocate (lk_looped_decode_step_static): a
// file-scope device array, one copy per GPU, which every such call on that GPU shares.
// Host code never passes `scratch` itself (on the host it is a stand-in, not a device
// address): each device's address comes from hipGetSymbolAddress, taken once per device
// with that device current, and the kernels receive that address.
constexpr size_t kStaticScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
    int dev = -1;
    LK_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(LK_ERR_UNSUPPORTED, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(LK_ERR_HIP, std::string("static scratch address: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LK_OK;
}

}  // namespace

extern "C" {

int lk_looped_decode_step(lk_handle* h, lk_kv_store* s, const int32_t* d_ids, float* d_out, void* d_ws,
                          size_t ws_bytes, void* stream) {
    if (!h || !s || !d_ids || !d_out || !d_ws) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (s->h != h) return fail(LK_ERR_INVALID_ARG, "store belongs to another handle");
    if (!s->prefilled) return fail(LK_ERR_STATE, "decode before prefill");
    if (s->t >= s->Tmax) return fail(LK_ERR_CAPACITY, "store is full (max_tokens reached)");
    const int B = s->B;
    const WS w = ws_layout(h, B, 1, (char*)d_ws);
    if (ws_bytes < w.total) return fail(LK_ERR_CAPACITY, "workspace too small");
    if ((uintptr_t)d_ws % kAlign) return fail(LK_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const int d = h->c.d_model;
    LK_HIP(hipMemcpyAsync(w.ids, d_ids, (size_t)B * 4, hipMemcpyDeviceToDevice, st));
    if (st && h->use_graphs) {
        DecodeGraph& g = h->graph;
        if (g.store != s || g.ws != d_ws || g.stream != st || g.timer_mask != (long long)h->timer.mask ||
            g.timer_per_call != h->timer.per_call || g.keep_codes != s->keep_codes) {
            g.reset();
            LK_TRY(capture_decode(h, s, w, st));
            g.store = s;
            g.ws = d_ws;
            g.stream = st;
            g.timer_mask = h->timer.mask;
            g.timer_per_call = h->timer.per_call;
            g.keep_codes = s->keep_codes;
        }
        for (const DecodeGraph::Seg& seg : g.segs) {
            if (seg.exec) {
                LK_HIP(hipGraphLaunch(seg.exec, st));
            } else {
                LK_HIP(h->timer.begin(st, seg.cls));
                LK_HIP(seg.direct());
                LK_HIP(h->timer.mark(st));
            }
        }
    } else {
        LK_TRY(enqueue_decode(h, s, w, st));
    }
    LK_HIP(hipMemcpyAsync(d_out, w.out, (size_t)B * d * 4, hipMemcpyDeviceToDevice, st));
    s->t += 1;
    return LK_OK;
}

int lk_looped_decode_step_static(lk_handle* h, lk_kv_store* s, const int32_t* d_ids, float* d_out, void* stream) {
    if (!h || !s || !d_ids || !d_out) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (s->h != h) return fail(LK_ERR_INVALID_ARG, "store belongs to another handle");
    if (!s->prefilled) return fail(LK_ERR_STATE, "decode before prefill");
    if (s->t >= s->Tmax) return fail(LK_ERR_CAPACITY, "store is full (max_tokens reached)");
    const int B = s->B;
    const size_t need = ws_layout(h, B, 1, nullptr).total;
    if (need > kStaticScratchBytes)
        return fail(LK_ERR_CAPACITY, "the decode workspace of this model and batch (" + std::to_string(need) +
                                         " bytes) exceeds the static scratch (" +
                                         std::to_string(kStaticScratchBytes) + " bytes)");
    void* ws = nullptr;
    LK_TRY(static_scratch(&ws));
    const WS w = ws_layout(h, B, 1, (char*)ws);
    hipStream_t st = (hipStream_t)stream;
    LK_HIP(hipMemcpyAsync(w.ids, d_ids, (size_t)B * 4, hipMemcpyDeviceToDevice, st));
    LK_TRY(enqueue_decode(h, s, w, st));
    LK_HIP(hipMemcpyAsync(d_out, w.out, (size_t)B * h->c.d_model * 4, hipMemcpyDeviceToDevice, st));
    s->t += 1;
    return LK_OK;
}

int lk_decode_weight_bytes(const lk_handle* h, size_t* bytes) {
    if (!h || !bytes) return fail(LK_ERR_INVALID_ARG, "null argument");
    *bytes = packed_weight_bytes(h);
    return LK_OK;
}

int lk_set_decode_weights(lk_handle* h, void* d_buf, size_t buf_bytes, void* stream) {
    if (!h) return fail(LK_ERR_INVALID_ARG, "null handle");
    h->graph.reset();
    if (!d_buf) {
        h->pk_buf = nullptr;
        h->PL.clear();
        return LK_OK;
    }
    const size_t need = packed_weight_bytes(h);
    if (!need) return fail(LK_ERR_UNSUPPORTED, "these shapes have no packed decode layout");
    if (buf_bytes < need) return fail(LK_ERR_CAPACITY, "decode weight buffer too small");
    if ((uintptr_t)d_buf % 16) return fail(LK_ERR_INVALID_ARG, "decode weight buffer must be 16-byte aligned");
    return pack_decode_weights(h, d_buf, (hipStream_t)stream);
}

int lk_set_decode_graphs(lk_handle* h, int32_t enable) {
    if (!h) return fail(LK_ERR_INVALID_ARG, "null handle");
    h->use_graphs = enable ? 1 : 0;
    h->graph.reset();
    return LK_OK;
}

int lk_timing_enable(lk_handle* h, const char* kernel_class) {
    if (!h) return fail(LK_ERR_INVALID_ARG, "null handle");
    unsigned mask = 0;
    if (kernel_class) {
        std::string list(kernel_class);
        size_t a = 0;
        while (a <= list.size()) {
            size_t b = list.find(',', a);
            if (b == std::string::npos) b = list.size();
            const std::string name = list.substr(a, b - a);
            int cls = TC_NONE;
            for (int i = 0; i < TC_COUNT; ++i)
                if (name == kTimedNames[i]) cls = i;
            if (cls == TC_NONE) return fail(LK_ERR_INVALID_ARG, "unknown kernel class " + name);
            mask |= 1u << cls;
            a = b + 1;
        }
    }
    h->timer.used = 0;
    h->timer.mask = mask;
    return LK_OK;
}

int lk_timing_sample(lk_handle* h, int32_t per_call) {
    if (!h || per_call < 0) return fail(LK_ERR_INVALID_ARG, "null handle or negative count");
    h->timer.per_call = per_call;
    return LK_OK;
}

namespace {
// Launches and summed event time of the recorded pairs of class cls (-1: every class).
int timing_sum(lk_handle* h, int cls, int32_t* launches, double* total_ms) {
    double tot = 0.0;
    int32_t n = 0;
    const size_t pairs = h->timer.used / 2;
    for (size_t i = 0; i < pairs; ++i) {
        if (cls >= 0 && h->timer.pair_cls[i] != cls) continue;
        LK_HIP(hipEventSynchronize(h->timer.pool[2 * i + 1]));
        float ms = 0.f;
        LK_HIP(hipEventElapsedTime(&ms, h->timer.pool[2 * i], h->timer.pool[2 * i + 1]));
        tot += ms;
        ++n;
    }
    *launches = n;
    *total_ms = tot;
    return LK_OK;
}
}  // namespace

int lk_timing_read(lk_handle* h, int32_t* launches, double* total_ms) {
    if (!h || !launches || !total_ms) return fail(LK_ERR_INVALID_ARG, "null argument");
    LK_TRY(timing_sum(h, -1, launches, total_ms));
    h->timer.used = 0;
    return LK_OK;
}

int lk_timing_read_class(lk_handle* h, const char* kernel_class, int32_t* launches, double* total_ms) {
    if (!h || !kernel_class || !launches || !total_ms) return fail(LK_ERR_INVALID_ARG, "null argument");
    int cls = TC_NONE;
    for (int i = 0; i < TC_COUNT; ++i)
        if (std::strcmp(kernel_class, kTimedNames[i]) == 0) cls = i;
    if (cls == TC_NONE) return fail(LK_ERR_INVALID_ARG, std::string("unknown kernel class ") + kernel_class);
    return timing_sum(h, cls, launches, total_ms);
}

// ---- test entry points ----------------------------------------------------------
int lk_dbg_topk(const float* d_keys, int32_t rows, int32_t cols, int32_t n, int32_t* d_idx, void* stream) {
    if (!d_keys || !d_idx) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (rows < 1 || cols < 1 || n < 1 || n > cols) return fail(LK_ERR_INVALID_ARG, "need 1 <= n <= cols");
    LK_HIP(lk::topk_rows(d_keys, rows, cols, n, d_idx, (hipStream_t)stream));
    return LK_OK;
}

int lk_dbg_quantize(const float* d_x, int32_t rows, int32_t hd, int32_t bits, uint8_t* d_codes,
                    uint16_t* d_scales, void* stream) {
    if (!d_x || !d_codes || !d_scales) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (rows < 1 || hd < 32 || hd % 32) return fail(LK_ERR_INVALID_ARG, "hd must be a positive multiple of 32");
    if (bits != 4 && bits != 8) return fail(LK_ERR_INVALID_ARG, "bits must be 4 or 8");
    LK_HIP(lk::quantize_rows(d_x, rows, hd, bits, d_codes, d_scales, (hipStream_t)stream));
    return LK_OK;
}

int lk_dbg_delta(const float* d_a, const float* d_b, int32_t rows, int32_t d, float* d_key, void* stream) {
    if (!d_a || !d_b || !d_key) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (rows < 1 || d < 1) return fail(LK_ERR_INVALID_ARG, "bad sizes");
    LK_HIP(lk::delta_keys(d_a, d_b, rows, d, d_key, (hipStream_t)stream));
    return LK_OK;
}

int lk_dbg_gemm(const void* d_a, const void* d_w, float* d_c, int32_t M, int32_t N, int32_t K, void* stream) {
    if (!d_a || !d_w || !d_c) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (M < 1 || N < 16 || N % 16 || K < 32 || K % 32)
        return fail(LK_ERR_INVALID_ARG, "need M >= 1, N a multiple of 16, K a multiple of 32");
    LK_HIP(lk::gemm((const u16*)d_a, (const u16*)d_w, M, N, K, lk::EPI_STORE, d_c, nullptr, (hipStream_t)stream));
    return LK_OK;
}

int lk_dbg_gemm_epi(const void* d_a, const void* d_w, int32_t epi, float* d_c, void* d_out, int32_t M, int32_t N,
                    int32_t K, void* stream) {
    if (!d_a || !d_w) return fail(LK_ERR_INVALID_ARG, "null argument");
    if (epi < lk::EPI_STORE || epi > lk::EPI_GELU) return fail(LK_ERR_INVALID_ARG, "epi must be 0..3");
    if (epi <= lk::EPI_ADD ? !d_c : !d_out) return fail(LK_ERR_INVALID_ARG, "null output for this epilogue");
    if (M < 1 || N < 16 || N % 16 || K < 32 || K % 32)
        return fail(LK_ERR_INVALID_ARG, "need M >= 1, N a multiple of 16, K a multiple of 32");
    LK_HIP(lk::gemm((const u16*)d_a, (const u16*)d_w, M, N, K, epi, d_c, (u16*)d_out, (hipStream_t)stream));
    return LK_OK;
}


int lk_dbg_attention(const lk_dbg_attn_args* x, size_t* ws_need, void* stream) {
    if (!x) return fail(LK_ERR_INVALID_ARG, "null argument");
    const int B = x->B, H = x->H, Hkv = x->Hkv, hd = x->hd;
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv) return fail(LK_ERR_INVALID_ARG, "bad head counts");
    const int G = H / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(LK_ERR_UNSUPPORTED, "H / Hkv must be 1, 2, 4 or 8");
    if (hd != 32 && hd != 64 && hd != 128) return fail(LK_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
    if (!x->q || !x->out) return fail(LK_ERR_INVALID_ARG, "null q or out");
    hipStream_t st = (hipStream_t)stream;
    auto rows_layer = [&](int fmt, const void* k, const void* v, const uint16_t* ks, const uint16_t* vs, int tmax) {
        KVLayer L{};
        L.B = B;
        L.Hkv = Hkv;
        L.hd = hd;
        L.Tmax = tmax;
        L.n_loops = 1;
        L.base[0] = k;
        L.base[1] = v;
        L.base_bits = 16;
        L.res_bits = 16;
        if (fmt == 1) {
            L.lazy = 1;
            L.base_bits = 8;
            L.base_scale[0] = ks;
            L.base_scale[1] = vs;
        } else if (fmt == 2) {
            L.f16 = 1;
        }
        return L;
    };
    size_t need = 0;
    switch (x->kind) {
        case LK_DBG_ATTN_DECODE:
        case LK_DBG_ATTN_DECODE_SEG: {
            lk::RowsAttn a{};
            a.q = (const u16*)x->q;
            a.q_half = x->q_half != 0;
            a.B = B;
            a.n_rows = 1;
            a.H = H;
            a.pos = x->t;
            a.k_loop = 1;
            a.out = (u16*)x->out;
            if (x->out32) {
                a.diff_mode = lk::DIFF_SET32;
                a.d32 = x->out32;
            }
            if (x->kind == LK_DBG_ATTN_DECODE) {
                if (x->kv_format != 0 && x->kv_format != 1) return fail(LK_ERR_UNSUPPORTED, "decode rows are bf16 or int8");
                if (!x->k || !x->v || (x->kv_format == 1 && (!x->k_scales || !x->v_scales)))
                    return fail(LK_ERR_INVALID_ARG, "null K/V rows");
                if (x->tmax < 8 || x->tmax % 8 || x->t < 0 || x->t >= x->tmax)
                    return fail(LK_ERR_INVALID_ARG, "need tmax a multiple of 8 and 0 <= t < tmax");
                a.kv = rows_layer(x->kv_format, x->k, x->v, x->k_scales, x->v_scales, x->tmax);
                // as a decode step: splits sized for the capacity tmax
                a.chunk = decode_dense_chunk((long long)B * Hkv, x->tmax);
                a.n_splits = (x->tmax + a.chunk - 1) / a.chunk;
            } else {
                if (!x->cols || !x->s_k || !x->s_v || !x->r_k || !x->r_v) return fail(LK_ERR_INVALID_ARG, "null argument");
                if (x->n_cols < 1 || x->s_cap < x->n_cols || x->s_cap % kSegChunk || x->r_cap % kSegChunk ||
                    x->window < 1 || x->r_cap < x->window + 8 || x->t < 0)
                    return fail(LK_ERR_INVALID_ARG, "need s_cap >= n_cols, s_cap and r_cap multiples of 128, "
                                                    "r_cap >= window + 8");
                a.kv = rows_layer(2, x->s_k, x->s_v, nullptr, nullptr, x->s_cap);
                a.kv2 = rows_layer(2, x->r_k, x->r_v, nullptr, nullptr, x->r_cap);
                a.cols = x->cols;
                a.n_cols = x->n_cols;
                a.window = x->window;
                a.chunk = kSegChunk;
                a.seg_split = x->s_cap / kSegChunk;
                a.n_splits = a.seg_split + x->r_cap / kSegChunk;
            }
            need = (size_t)B * H * a.n_splits * (hd + 2) * 4;
            if (!x->ws) {
                if (ws_need) break;
                return fail(LK_ERR_INVALID_ARG, "null workspace");
            }
            if (x->ws_bytes < need) return fail(LK_ERR_CAPACITY, "workspace too small");
            a.part = (float*)x->ws;
            LK_HIP(lk::attn_rows_main(a, st));
            LK_HIP(lk::attn_rows_combine(a, st, false));
            break;
        }
        case LK_DBG_ATTN_PREFILL:
        case LK_DBG_ATTN_MASS: {
            if (x->kv_format != 0 && x->kv_format != 1) return fail(LK_ERR_UNSUPPORTED, "prefill rows are bf16 or int8");
            if (!x->k || !x->v || (x->kv_format == 1 && (!x->k_scales || !x->v_scales)) || !x->lse)
                return fail(LK_ERR_INVALID_ARG, "null argument");
            if (x->kind == LK_DBG_ATTN_MASS && !x->mass) return fail(LK_ERR_INVALID_ARG, "null mass");
            if (x->T < 1 || x->tmax < x->T || x->tmax % 8) return fail(LK_ERR_INVALID_ARG, "need 1 <= T <= tmax, tmax % 8 == 0");
            if (!x->ws && ws_need) break;
            const KVLayer L = rows_layer(x->kv_format, x->k, x->v, x->k_scales, x->v_scales, x->tmax);
            if (x->kind == LK_DBG_ATTN_PREFILL)
                LK_HIP(lk::attn_prefill((const u16*)x->q, L, B, x->T, H, (u16*)x->out, x->lse, st));
            else
                LK_HIP(lk::column_mass((const u16*)x->q, L, x->lse, B, x->T, H, x->mass, st));
            break;
        }
        case LK_DBG_ATTN_PREFILL_SPARSE: {
            if (hd != 128) return fail(LK_ERR_UNSUPPORTED, "the sparse prefill rows take head_dim 128");
            if (!x->cols || !x->qpos || !x->s_k || !x->s_v || !x->r_k || !x->r_v) return fail(LK_ERR_INVALID_ARG, "null argument");
            if (x->n_rows < 1 || x->n_cols < 1 || x->window < 1 || x->s_cap < x->n_cols || x->s_cap % 8 || x->r_cap % 8)
                return fail(LK_ERR_INVALID_ARG, "bad sizes");
            if (!x->ws && ws_need) break;
            lk::RowsAttn a{};
            a.q = (const u16*)x->q;
            a.qpos = x->qpos;
            a.B = B;
            a.n_rows = x->n_rows;
            a.H = H;
            a.cols = x->cols;
            a.n_cols = x->n_cols;
            a.window = x->window;
            a.out = (u16*)x->out;
            a.kv = rows_layer(2, x->s_k, x->s_v, nullptr, nullptr, x->s_cap);
            const KVLayer fr = rows_layer(2, x->r_k, x->r_v, nullptr, nullptr, x->r_cap);
            LK_HIP(lk::attn_rows_prefill(a, a.kv, fr, st));
            break;
        }
        default:
            return fail(LK_ERR_INVALID_ARG, "unknown kind");
    }
    if (ws_need) *ws_need = need;
    return LK_OK;
}

int lk_dbg_kv_write(lk_kv_store* s, int32_t layer, int32_t loop, const float* d_qkv, int32_t rows_per_seq,
                    const int32_t* d_pos, void* d_q_out, int32_t q_half, void* d_ws, size_t ws_bytes, void* stream) {
    if (!s || !d_qkv || !d_q_out) return fail(LK_ERR_INVALID_ARG, "null argument");
    lk_handle* h = s->h;
    if (!h->lazy()) return fail(LK_ERR_UNSUPPORTED, "the writer test entry takes lazy stores");
    const lk_model_cfg& c = h->c;
    if (layer < 0 || layer >= c.n_shared || loop < 1 || loop > s->K) return fail(LK_ERR_INVALID_ARG, "bad layer or loop");
    hipStream_t st = (hipStream_t)stream;
    const int B = s->B;
    lk::KVWrite kw{};
    kw.layer = lazy_layer(s, layer);
    kw.loop = loop;
    kw.kind = loop == 1 ? 1 : 2;
    kw.keep_codes = 0;
    kw.range_flag = range_flag(s);
    if (d_pos) {
        if (rows_per_seq < 1 || rows_per_seq > s->Tpad || (loop >= 2 && rows_per_seq > s->lay.slots))
            return fail(LK_ERR_INVALID_ARG, "rows_per_seq out of range");
        kw.slot_base = 0;
        if (loop >= 2) kw.slot_map_k = slot_map(s, loop);
        LK_HIP(lk::rope_kv_write(d_qkv, B * rows_per_seq, rows_per_seq, d_pos, 0, c.n_heads, c.n_kv_heads, c.head_dim,
                                 h->inv_freq, (u16*)d_q_out, kw, st, q_half));
        return LK_OK;
    }
    if (!s->prefilled) return fail(LK_ERR_STATE, "decode-mode write before prefill");
    if (s->t >= s->Tmax) return fail(LK_ERR_CAPACITY, "store is full");
    if (!d_ws) return fail(LK_ERR_INVALID_ARG, "decode mode needs the decode workspace");
    const WS w = ws_layout(h, B, 1, (char*)d_ws);
    if (ws_bytes < w.total) return fail(LK_ERR_CAPACITY, "workspace too small");
    const int32_t* dpos = dev_pos(s);
    LK_HIP(lk::rope_angles(dpos, h->inv_freq, c.head_dim, w.rope, st));
    kw.dpos = dpos;
    kw.rope_cs = w.rope;
    kw.tok_recon = w.tokrec + (long long)layer * B * 2 * c.n_kv_heads * c.head_dim;
    if (loop >= 2) {
        kw.ring = scache_layer(s, loop, layer, true);
        kw.ring_on = 1;
        kw.slot_base = (long long)loop_rows(s, loop) - s->Tp;
        kw.slot_map_k = slot_map(s, loop);
    }
    LK_HIP(lk::rope_kv_write(d_qkv, B, 1, nullptr, 0, c.n_heads, c.n_kv_heads, c.head_dim, h->inv_freq,
                             (u16*)d_q_out, kw, st, q_half));
    return LK_OK;
}

}  // extern "C"
