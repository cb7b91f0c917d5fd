// Attention kernels for gfx950.
//
// The sparse path follows the FlashLoop abstract (arxivdaily.com): attention
// output differences across loops are dominated by a sparse, stable subset of
// key columns, so loops k >= 2 attend over that subset plus a recent window,
// reading a KV that is the previous loop's plus quantized residuals.
//
// Scores are kept in log2 units (q.k * log2(e) / sqrt(hd)) everywhere, so that the
// split partials (m, l, o) of every kernel combine the same way.
//
// * attn_prefill: causal flash attention with v_mfma_f32_32x32x16 (bf16 operands over
//   bf16 rows; float16 over int8 rows, whose codes times scales are rounded once).  Scores
//   are formed transposed (S^T = K Q^T) so every lane owns one query column and
//   the softmax statistics stay per lane (lanes l and l+32 share a query).  The
//   K rows of a tile are staged in LDS in a permuted order chosen so that each
//   lane's score accumulators cover 8 consecutive keys per 16-key step; those
//   accumulators are then directly the P^T operand of O^T = V^T P^T, and the V^T
//   operand is one 16-byte LDS read out of the 8-key-interleaved V tile.
// * column_mass: the per-column sum of the loop-1 softmax probabilities, keys
//   outer / queries inner, so each column is reduced in one fixed order.
// * attn_decode_dense: one query token over contiguous rows (base / dense
//   caches), split over the context.  v_mfma_f32_16x16x32 (f16 for int8 rows,
//   bf16 for bf16 rows) with both operands loaded straight from HBM: K rows for
//   S^T = K Q^T, the 8-key-interleaved V for O^T = V^T P^T.  int8 codes become
//   f16 with a byte-permute "magic number" conversion and are scaled by their
//   float16 group scales in packed f16.
// * attn_rows: query rows over explicit sparse column sets (decode loops >= 2
//   and kept prefill tokens); reconstructs K/V from the store in fp32 (base +
//   loop residuals); lanes own keys for q.k and head dims for p.V.
#include "lk_kernels.h"

namespace lk {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// Operand type of the prefill kernels: float16 over int8 rows (code * scale rounded
// once to float16; q converted from bf16) and bf16 over bf16 rows.  Eight operand
// elements travel as one uint4.  The float16 forms assume magnitudes inside the float16
// range: a bf16 q above 65504 or an int8 element (code * scale) above it becomes inf, and
// bf16 values below 2^-14 lose bits as float16 subnormals.
template <bool F16>
__device__ __forceinline__ uint32_t pack_op2(float a, float b) {
    if constexpr (F16) return pack_h2(a, b);
    else return pack_bf2(a, b);
}
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    if constexpr (F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(a), as_half8(b), c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// Eight bf16 values as float16: exact for magnitudes in [2^-14, 65504]; larger ones
// become inf, smaller ones float16 subnormals.
__device__ __forceinline__ uint4 bf8_to_h8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o[t] = pack_h2(__uint_as_float(w[t] << 16), __uint_as_float(w[t] & 0xFFFF0000u));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8 signed bytes -> 8 float16 (exact), multiplied by per-pair scales (packed f16).
// Byte j of the input becomes element j.  Each byte is biased to u = c + 128 and
// placed under the float16 exponent of 1024 (bits 0x64uu = 1024 + u); subtracting
// 1152 leaves c exactly.
__device__ __forceinline__ uint4 i8x8_to_f16(uint2 c, uint4 scale_pairs) {
    const uint32_t u0 = c.x ^ 0x80808080u, u1 = c.y ^ 0x80808080u;
    uint32_t w[4];
    w[0] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u);
    w[1] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u);
    w[2] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u);
    w[3] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u);
    const uint32_t sc[4] = {scale_pairs.x, scale_pairs.y, scale_pairs.z, scale_pairs.w};
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        half2v h = __builtin_bit_cast(half2v, w[j]) - bias;
        h = h * __builtin_bit_cast(half2v, sc[j]);
        o[j] = __builtin_bit_cast(uint32_t, h);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8 consecutive K elements of row (b, g, pos) as operands: bf16 rows as they are, int8
// codes times their group scale as float16 (the exact product rounded once).
template <int HD, bool I8>
__device__ __forceinline__ uint4 load_k8(const KVLayer& kv, int b, int g, int pos, int e0) {
    const long long row = kv_row(kv, b, g, pos);
    if (!I8) return *(const uint4*)((const u16*)kv.base[0] + row * HD + e0);
    const uint2 c = *(const uint2*)((const int8_t*)kv.base[0] + row * HD + e0);
    const uint32_t s2 = (uint32_t)kv.base_scale[0][row * (HD / 32) + e0 / 32] * 0x10001u;
    return i8x8_to_f16(c, make_uint4(s2, s2, s2, s2));
}

// Zero the bf16/f16 elements j >= valid of an 8-element operand.
__device__ __forceinline__ uint4 mask_tail8(uint4 v, int valid) {
    if (valid >= 8) return v;
    uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (2 * q >= valid) o[q] &= 0xFFFF0000u;
        if (2 * q + 1 >= valid) o[q] &= 0x0000FFFFu;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Eight keys [pos0, pos0+8) of V at head dim e as operands (pos0 a multiple of 8; bf16
// rows, or int8 codes times scales as float16), keys >= valid zeroed.
template <int HD, bool I8>
__device__ __forceinline__ uint4 load_v8(const KVLayer& kv, int b, int g, int pos0, int e, int valid) {
    const long long idx = v_elem(kv, b, g, pos0, e);
    uint4 out;
    if (!I8) {
        out = *(const uint4*)((const u16*)kv.base[1] + idx);
    } else {
        const uint2 c = *(const uint2*)((const int8_t*)kv.base[1] + idx);
        // the scales of keys pos0..pos0+7 in this 32-wide group are 8 consecutive float16
        out = i8x8_to_f16(c, *(const uint4*)(kv.base_scale[1] + v_scale_idx(kv, b, g, pos0, e / 32)));
    }
    return mask_tail8(out, valid);
}

// ---------------------------------------------------------------- flash prefill
// Key held by LDS row r of a 32-key K tile: lane group kg of the 32x32 score
// accumulator then owns keys 8kg..8kg+7 (accumulators 0..7) and 16+8kg.. (8..15).
__device__ __forceinline__ int flash_key_of_row(int r) {
    const int a = r >> 3;
    return ((a >= 2) ? 16 : 0) + 8 * ((r >> 2) & 1) + 4 * (a & 1) + (r & 3);
}

template <int HD, bool I8>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const u16* __restrict__ Q, KVLayer kv,
                                                           int T, int H, u16* __restrict__ O,
                                                           float* __restrict__ LSE, float sl2) {
    constexpr int KT = 32;
    constexpr int LDK = HD + 8;       // K tile row (keys x hd)
    constexpr int LDV = KT + 8;       // V^T tile row (hd x keys)
    constexpr int CPR = HD / 8;
    constexpr int NKC = KT * CPR;     // 16-byte K chunks per tile
    constexpr int NVC = (KT / 8) * HD;  // 16-byte V chunks per tile (8 keys x one e)
    constexpr int PER = (NKC + NVC + 255) / 256;
    __shared__ __attribute__((aligned(16))) u16 Ks[2][KT * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[2][HD * LDV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kg = lane >> 5, l32 = lane & 31;
    const int h = blockIdx.y, b = blockIdx.z;
    const int G = H / kv.Hkv, g = h / G;
    const int qblk = blockIdx.x * 128;
    const int q0 = qblk + w * 32;
    const int qi = q0 + l32;
    const long long ldq = (long long)H * HD;

    uint4 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qi < T) v = *(const uint4*)(Q + ((long long)b * T + qi) * ldq + h * HD + ks * 16 + kg * 8);
        qf[ks] = I8 ? bf8_to_h8(v) : v;
    }
    f32x16 oacc[HD / 32];
#pragma unroll
    for (int c = 0; c < HD / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
    float m_i = -INFINITY, l_i = 0.f;

    const int kend = min(T, qblk + 128);
    const int ntiles = (kend + KT - 1) / KT;
    uint4 regs[PER];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * 256;
            regs[p] = make_uint4(0, 0, 0, 0);
            if (c < NKC) {
                const int key = t * KT + flash_key_of_row(c / CPR);
                if (key < T) regs[p] = load_k8<HD, I8>(kv, b, g, key, (c % CPR) * 8);
            } else if (c < NKC + NVC) {
                const int cc = c - NKC;
                const int blk = cc / HD, e = cc % HD;
                const int pos0 = t * KT + blk * 8;
                if (pos0 < T) regs[p] = load_v8<HD, I8>(kv, b, g, pos0, e, T - pos0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * 256;
            if (c < NKC) {
                *(uint4*)&Ks[buf][(c / CPR) * LDK + (c % CPR) * 8] = regs[p];
            } else if (c < NKC + NVC) {
                const int cc = c - NKC;
                *(uint4*)&Vt[buf][(cc % HD) * LDV + (cc / HD) * 8] = regs[p];
            }
        }
    };
    load_tile(0);
    store_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);
        const int kbase = t * KT;
        if (kbase <= q0 + 31) {
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < HD / 16; ++ks) {
                s = mfma32<I8>(*(const uint4*)&Ks[cur][l32 * LDK + ks * 16 + kg * 8], qf[ks], s);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kbase + ((i < 8) ? 8 * kg + i : 16 + 8 * kg + (i - 8));
                const float v = (key <= qi && key < T) ? s[i] * sl2 : -INFINITY;
                s[i] = v;
                mx = fmaxf(mx, v);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_i, mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_i - m_new);
            float p[16];
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = (s[i] == -INFINITY) ? 0.f : exp2f(s[i] - m_new);
                rs += p[i];
            }
            rs += __shfl_xor(rs, 32);
            l_i = l_i * alpha + rs;
            m_i = m_new;
#pragma unroll
            for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
            uint4 pb0, pb1;
            pb0.x = pack_op2<I8>(p[0], p[1]);
            pb0.y = pack_op2<I8>(p[2], p[3]);
            pb0.z = pack_op2<I8>(p[4], p[5]);
            pb0.w = pack_op2<I8>(p[6], p[7]);
            pb1.x = pack_op2<I8>(p[8], p[9]);
            pb1.y = pack_op2<I8>(p[10], p[11]);
            pb1.z = pack_op2<I8>(p[12], p[13]);
            pb1.w = pack_op2<I8>(p[14], p[15]);
#pragma unroll
            for (int c = 0; c < HD / 32; ++c) {
                const u16* vrow = &Vt[cur][(c * 32 + l32) * LDV];
                oacc[c] = mfma32<I8>(*(const uint4*)(vrow + 8 * kg), pb0, oacc[c]);
                oacc[c] = mfma32<I8>(*(const uint4*)(vrow + 16 + 8 * kg), pb1, oacc[c]);
            }
        }
        if (t + 1 < ntiles) store_tile(cur ^ 1);
    }
    if (qi < T) {
        const float inv = 1.f / l_i;
        u16* orow = O + ((long long)b * T + qi) * ldq + h * HD;
#pragma unroll
        for (int c = 0; c < HD / 32; ++c)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e0 = c * 32 + 8 * i4 + 4 * kg;
                uint2 v;
                v.x = pack_bf2(oacc[c][i4 * 4 + 0] * inv, oacc[c][i4 * 4 + 1] * inv);
                v.y = pack_bf2(oacc[c][i4 * 4 + 2] * inv, oacc[c][i4 * 4 + 3] * inv);
                *(uint2*)(orow + e0) = v;
            }
        if (kg == 0) LSE[((long long)b * H + h) * T + qi] = m_i + log2f(l_i);
    }
}

// ---------------------------------------------------------------- flash prefill, hd 128
// 64-key tiles, one head and 32 NW queries per workgroup (NW waves x 32 queries), K/V
// staged through registers into double-buffered LDS.  S^T = K Q^T for each 32-key half
// (LDS rows permuted by flash_key_of_row so the score accumulator is already the B
// operand of O^T += V^T P^T).  Per tile and lane: one FMA and one v_exp_f32 per score;
// the output is rescaled only when some query's running max grows (a wave-uniform
// branch); tiles below the diagonal skip the causal mask.  Workgroups take query blocks
// from the last one down, so the longest causal spans start first.
//
// NW 4: each thread stages 8 of a tile's 16-byte chunks, one tile ahead.  NW 8: each
// thread stages 4 chunks, into two register sets in turn, so a tile's loads are issued
// two tiles before it is stored to LDS (the same registers as NW 4, twice the time to
// land).
template <bool I8, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_prefill_fa_kernel(const u16* __restrict__ Q, KVLayer kv,
                                                                           int T, int H, u16* __restrict__ O,
                                                                           float* __restrict__ LSE, float sl2) {
    constexpr int HD = 128, KT = 64, NT = 64 * NW;
    constexpr int LDK = HD + 8;
    constexpr int LDV = KT + 8;
    constexpr int CPR = HD / 8;             // 16-byte chunks per K row
    constexpr int NKC = KT * CPR;           // 1024 K chunks per tile
    constexpr int NVC = (KT / 8) * HD;      // 1024 V chunks per tile
    constexpr int PER = (NKC + NVC) / NT;   // chunks per thread
    constexpr int PK = NKC / NT;            // of which K chunks
    __shared__ __attribute__((aligned(16))) u16 Ks[2][KT * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[2][HD * LDV];
    // the wave index through readfirstlane: the per-wave tests below (a tile above the
    // wave's queries, a tile that needs the causal mask) are then scalar branches, not
    // lane-masked regions that every tile would step through
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, l32 = lane & 31;
    // workgroups of one sequence in order of causal work: every head's last query
    // block, then every head's second last, ... (the dispatch runs x, then y)
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int h = lin % gridDim.y, b = blockIdx.z;
    const int G = H / kv.Hkv, g = h / G;
    const int qblk = (gridDim.x - 1 - lin / gridDim.y) * (32 * NW);
    const int q0 = qblk + w * 32;
    const int qi = q0 + l32;
    const long long ldq = (long long)H * HD;

    uint4 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qi < T) v = *(const uint4*)(Q + ((long long)b * T + qi) * ldq + h * HD + ks * 16 + kg * 8);
        qf[ks] = I8 ? bf8_to_h8(v) : v;
    }
    f32x16 oacc[HD / 32];
#pragma unroll
    for (int c = 0; c < HD / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
    float m_i = -INFINITY, l_i = 0.f;

    const int kend = min(T, qblk + 32 * NW);
    const int ntiles = (kend + KT - 1) / KT;
    // A tile whose 64 keys all lie below T is loaded without bounds checks: K chunk p of
    // this thread (LDS row tid/16 + (NT/16) p) holds key k0 + (NT/16) p of the tile, V
    // chunk p the 8 keys of V block tid/128 + (NT/128) (p - PK) at head dim tid % 128, so
    // every address is a fixed per-thread offset plus the tile's row offset, which the
    // whole workgroup shares.  Only a last partial tile takes the checked loads.
    const long long row0 = (long long)(b * kv.Hkv + g) * kv.Tmax;
    const int k0 = flash_key_of_row(tid / CPR);
    const int koff = k0 * HD + (tid % CPR) * 8;                              // elements
    const int ksoff = k0 * (HD / 32) + (tid % CPR) / 4;                      // K scale index
    const int voff = (tid / HD) * HD * 8 + (tid % HD) * 8;                   // elements
    const int vsoff = ((tid / HD) * (HD / 32) + (tid % HD) / 32) * 8;        // V scale index
    auto load_tile = [&](uint4 (&regs)[PER], int t) {
        if ((t + 1) * KT <= T) {
            const long long r = row0 + (long long)t * KT;
            if constexpr (I8) {
                const int8_t* kc = (const int8_t*)kv.base[0] + r * HD;
                const int8_t* vc = (const int8_t*)kv.base[1] + r * HD;
                const u16* ks = kv.base_scale[0] + r * (HD / 32);
                const u16* vs = kv.base_scale[1] + r * (HD / 32);
#pragma unroll
                for (int p = 0; p < PK; ++p) {
                    const uint32_t s2 = (uint32_t)ks[ksoff + p * (NT / 16) * (HD / 32)] * 0x10001u;
                    regs[p] = i8x8_to_f16(*(const uint2*)(kc + koff + p * (NT / 16) * HD), make_uint4(s2, s2, s2, s2));
                }
#pragma unroll
                for (int p = 0; p < PER - PK; ++p)
                    regs[PK + p] = i8x8_to_f16(*(const uint2*)(vc + voff + p * NT * 8),
                                               *(const uint4*)(vs + vsoff + p * (NT / HD) * (HD / 32) * 8));
            } else {
                const u16* kb = (const u16*)kv.base[0] + r * HD;
                const u16* vb = (const u16*)kv.base[1] + r * HD;
#pragma unroll
                for (int p = 0; p < PK; ++p) regs[p] = *(const uint4*)(kb + koff + p * (NT / 16) * HD);
#pragma unroll
                for (int p = 0; p < PER - PK; ++p) regs[PK + p] = *(const uint4*)(vb + voff + p * NT * 8);
            }
            return;
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            regs[p] = make_uint4(0, 0, 0, 0);
            if (c < NKC) {
                const int r = c / CPR;
                const int key = t * KT + (r & 32) + flash_key_of_row(r & 31);
                if (key < T) regs[p] = load_k8<HD, I8>(kv, b, g, key, (c % CPR) * 8);
            } else {
                const int cc = c - NKC;
                const int blk = cc / HD, e = cc % HD;
                const int pos0 = t * KT + blk * 8;
                if (pos0 < T) regs[p] = load_v8<HD, I8>(kv, b, g, pos0, e, T - pos0);
            }
        }
    };
    auto store_tile = [&](const uint4 (&regs)[PER], int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            if (c < NKC) {
                *(uint4*)&Ks[buf][(c / CPR) * LDK + (c % CPR) * 8] = regs[p];
            } else {
                const int cc = c - NKC;
                *(uint4*)&Vt[buf][(cc % HD) * LDV + (cc / HD) * 8] = regs[p];
            }
        }
    };
    // one tile from LDS buffer cur: scores, online softmax, P V
    auto attend_tile = [&](int t, int cur) {
        const int kbase = t * KT;
        if (kbase > q0 + 31) return;
        f32x16 sc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[hh][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < HD / 16; ++ks) {
                sc[hh] = mfma32<I8>(*(const uint4*)&Ks[cur][(32 * hh + l32) * LDK + ks * 16 + kg * 8], qf[ks], sc[hh]);
            }
        }
        // causal / length mask only where the tile reaches the diagonal or the end
        const bool full = kbase + KT - 1 <= q0 && kbase + KT <= T;
        if (!full) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kbase + 32 * hh + ((i < 8) ? 8 * kg + i : 16 + 8 * kg + (i - 8));
                    if (key > qi || key >= T) sc[hh][i] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[hh][i]);
        {  // the row's other half sits 32 lanes away: exchange the halves in registers
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        const float m_new = fmaxf(m_i, mx * sl2);
        if (__builtin_amdgcn_ballot_w64(m_new > m_i)) {
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_i - m_new);
            l_i *= alpha;
#pragma unroll
            for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
        }
        m_i = m_new;
        const float nm = -m_new;
        float rs = 0.f;
        uint4 pb[2][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = __builtin_amdgcn_exp2f(fmaf(sc[hh][i], sl2, nm));
                rs += p[i];
            }
            uint4 pu0, pu1;
            pu0.x = pack_op2<I8>(p[0], p[1]);
            pu0.y = pack_op2<I8>(p[2], p[3]);
            pu0.z = pack_op2<I8>(p[4], p[5]);
            pu0.w = pack_op2<I8>(p[6], p[7]);
            pu1.x = pack_op2<I8>(p[8], p[9]);
            pu1.y = pack_op2<I8>(p[10], p[11]);
            pu1.z = pack_op2<I8>(p[12], p[13]);
            pu1.w = pack_op2<I8>(p[14], p[15]);
            pb[hh][0] = pu0;
            pb[hh][1] = pu1;
        }
        l_i += rs;  // this lane's half of the row sum; the halves are added once at the end
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < HD / 32; ++c) {
                const u16* vrow = &Vt[cur][(c * 32 + l32) * LDV + 32 * hh];
                oacc[c] = mfma32<I8>(*(const uint4*)(vrow + 8 * kg), pb[hh][0], oacc[c]);
                oacc[c] = mfma32<I8>(*(const uint4*)(vrow + 16 + 8 * kg), pb[hh][1], oacc[c]);
            }
    };
    if constexpr (NW == 4) {
        uint4 regs[PER];
        load_tile(regs, 0);
        store_tile(regs, 0);
        for (int t = 0; t < ntiles; ++t) {
            const int cur = t & 1;
            __syncthreads();
            if (t + 1 < ntiles) load_tile(regs, t + 1);
            attend_tile(t, cur);
            if (t + 1 < ntiles) store_tile(regs, cur ^ 1);
        }
    } else {
        // tile t sits in LDS buffer t & 1; register set A carries the odd tiles, B the
        // even ones from tile 2 on, each loaded two tiles before it is stored
        uint4 ra[PER], rb[PER];
        load_tile(ra, 0);
        store_tile(ra, 0);
        if (ntiles > 1) load_tile(ra, 1);
        if (ntiles > 2) load_tile(rb, 2);
        for (int t = 0; t < ntiles; t += 2) {
            __syncthreads();
            attend_tile(t, 0);
            if (t + 1 < ntiles) store_tile(ra, 1);
            if (t + 3 < ntiles) load_tile(ra, t + 3);
            if (t + 1 >= ntiles) break;
            __syncthreads();
            attend_tile(t + 1, 1);
            if (t + 2 < ntiles) store_tile(rb, 0);
            if (t + 4 < ntiles) load_tile(rb, t + 4);
        }
    }
    l_i += __shfl_xor(l_i, 32);
    if (qi < T) {
        const float inv = 1.f / l_i;
        u16* orow = O + ((long long)b * T + qi) * ldq + h * HD;
#pragma unroll
        for (int c = 0; c < HD / 32; ++c)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e0 = c * 32 + 8 * i4 + 4 * kg;
                uint2 v;
                v.x = pack_bf2(oacc[c][i4 * 4 + 0] * inv, oacc[c][i4 * 4 + 1] * inv);
                v.y = pack_bf2(oacc[c][i4 * 4 + 2] * inv, oacc[c][i4 * 4 + 3] * inv);
                *(uint2*)(orow + e0) = v;
            }
        if (kg == 0) LSE[((long long)b * H + h) * T + qi] = m_i + log2f(l_i);
    }
}

// ---------------------------------------------------------------- column mass
// mass[b, g, j] = sum over the group's heads h and queries q >= j of 2^(s_qj sl2 - lse_qh).
// NW waves per workgroup, 32 keys each, K held in registers as the A operand.  The query
// tiles (one head and 32 queries at a time) stream through double-buffered LDS, the next
// tile's global loads issued before the current tile's products; every staged tile serves
// 32 NW keys.  Per score: one FMA, one v_exp_f32 and one add; the causal mask is applied only
// on tiles that reach the diagonal.
template <int HD, bool I8, int NW, int QS>
__global__ __launch_bounds__(64 * NW) void column_mass_kernel(const u16* __restrict__ Q, KVLayer kv,
                                                              const float* __restrict__ LSE, int T, int H,
                                                              float* __restrict__ mass, float sl2) {
    constexpr int LDQ = HD + 8;
    constexpr int CPR = HD / 8;
    constexpr int QR = 32 * QS;    // query rows per staged tile (QS MFMA tiles of 32)
    constexpr int NQC = QR * CPR;  // 16-byte chunks of one query tile
    constexpr int NT = 64 * NW;
    constexpr int PER = (NQC + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) u16 Qs[2][QR * LDQ];
    // wave index through readfirstlane: the diagonal tests are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, l32 = lane & 31;
    // workgroups of one sequence in order of causal work: every KV head's first key
    // block (all queries see it), then every head's second, ... (the dispatch runs x, then y)
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int g = lin % gridDim.y, b = blockIdx.z;
    const int Hkv = kv.Hkv, G = H / Hkv;
    const int kblk = (lin / gridDim.y) * 32 * NW;
    const int j0 = kblk + w * 32;
    const long long ldq = (long long)H * HD;
    uint4 kf[HD / 16];
    {
        const int key = j0 + l32;
#pragma unroll
        for (int ks = 0; ks < HD / 16; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key < T) v = load_k8<HD, I8>(kv, b, g, key, ks * 16 + kg * 8);
            kf[ks] = v;
        }
    }
    float cs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cs[i] = 0.f;
    // The loop walks (head hh, query tile qt) with qt fastest, from the tile holding the
    // workgroup's first key to the last one.  Query chunk p of this thread is row
    // tid/16 + (NT/16) p of the tile at elements (tid % 16) 8: a fixed offset from the
    // tile's first row; a full tile loads without bounds checks.
    const int qt0 = kblk / QR, nqt = (T + QR - 1) / QR, nit = G * (nqt - qt0);
    const int qr = tid / CPR;
    const long long qoff = (long long)qr * ldq + (tid % CPR) * 8;
    uint4 regs[PER];
    auto load_tile = [&](int hh, int qt) {
        const u16* qb = Q + ((long long)b * T + qt * QR) * ldq + (g * G + hh) * HD;
        const bool full = qt * QR + QR <= T;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            regs[p] = make_uint4(0, 0, 0, 0);
            if (tid + p * NT < NQC && (full || qt * QR + qr + p * (NT / CPR) < T))
                regs[p] = *(const uint4*)(qb + qoff + (long long)p * (NT / CPR) * ldq);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            if (c < NQC) *(uint4*)&Qs[buf][(c / CPR) * LDQ + (c % CPR) * 8] = I8 ? bf8_to_h8(regs[p]) : regs[p];
        }
    };
    int hh = 0, qt = qt0;  // the tile in LDS buffer it & 1
    load_tile(hh, qt);
    store_tile(0);
    for (int it = 0; it < nit; ++it) {
        const int cur = it & 1;
        int hn = hh, qn = qt + 1;
        if (qn == nqt) {
            qn = qt0;
            ++hn;
        }
        __syncthreads();
        if (it + 1 < nit) load_tile(hn, qn);
        const int h = g * G + hh;
#pragma unroll
        for (int sq = 0; sq < QS; ++sq) {
            const int q0 = qt * QR + sq * 32, q = q0 + l32;
            if (q0 + 31 < j0) continue;
            const float lse2 = (q < T) ? LSE[((long long)b * H + h) * T + q] : 0.f;
            f32x16 sv;
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < HD / 16; ++ks)
                sv = mfma32<I8>(kf[ks], *(const uint4*)&Qs[cur][(sq * 32 + l32) * LDQ + ks * 16 + kg * 8], sv);
            if (q0 >= j0 + 31) {  // every key of this wave precedes every query of the tile
                if (q < T) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) cs[i] += __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -lse2));
                }
            } else if (q < T) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j0 + 8 * (i >> 2) + 4 * kg + (i & 3);
                    if (key <= q) cs[i] += __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -lse2));
                }
            }
        }
        if (it + 1 < nit) store_tile(cur ^ 1);
        hh = hn;
        qt = qn;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float v = cs[i];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
        cs[i] = v;
    }
    if (l32 == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = j0 + 8 * (i >> 2) + 4 * kg + (i & 3);
            if (key < T) mass[((long long)b * Hkv + g) * T + key] = cs[i];
        }
    }
}

// ---------------------------------------------------------------- dense decode (MFMA)
// Row types of the dense decode kernel.
// RT_F16_2SEG_LIVE: two segments, and the launch stops after the new token's K/V write
// when no sequence is left in the loops (*a.live == 0).
enum { RT_BF16 = 0, RT_I8 = 1, RT_F16 = 2, RT_F16_2SEG = 3, RT_F16_2SEG_LIVE = 4 };

// One 32-key tile [kb, kb + 32) of the decode attention for the wave that calls it: keys
// in [c_lo, c_end) take part, row_of(key) is the key's row in kv.  Lane (kgrp, head c16)
// holds the Q^T operand qop and the wave's running max m, sum l and O^T tiles oacc.
template <int HD, int G, int RT, class RowOf>
__device__ __forceinline__ void decode_tile(const KVLayer& kv, int b, int g, int kb, int c_lo, int c_end,
                                            RowOf row_of, const uint4 (&qop)[HD / 32], f32x4 (&oacc)[HD / 16],
                                            float& m, float& l, float sl2, int c16, int kgrp) {
    constexpr bool I8 = RT == RT_I8;
    constexpr bool HALF = RT != RT_BF16;  // f16 MFMA (int8 codes are converted to f16)
    constexpr int NQ = HD / 32;
    constexpr int NE = HD / 16;
    constexpr bool KPERM = I8 && NQ % 2 == 0;
    // V operands of the tile are loaded first, so that K and V are in flight together.
    // int8 V: one 16-byte load per pair of O^T tiles; tile et's row r is head dim
    // vdim(et, r) = 32 (et/2) + 2 r + et%2 (the 8 keys of dims e and e + 1 are adjacent)
    const int pos0 = row_of(min(kb + 8 * kgrp, ((c_end - 1) >> 3) << 3));
    uint4 vraw[I8 ? NE / 2 : NE], vsc[I8 ? NE / 2 : 1];
    if (I8) {
#pragma unroll
        for (int pp = 0; pp < NE / 2; ++pp) {
            vraw[pp] = *(const uint4*)((const int8_t*)kv.base[1] + v_elem(kv, b, g, pos0, 32 * pp + 2 * c16));
            vsc[pp] = *(const uint4*)(kv.base_scale[1] + v_scale_idx(kv, b, g, pos0, pp));
        }
    } else {
#pragma unroll
        for (int et = 0; et < NE; ++et) vraw[et] = *(const uint4*)((const u16*)kv.base[1] + v_elem(kv, b, g, pos0, 16 * et + c16));
    }
    // ---- S^T = K Q^T: n-tile nt covers keys kb + 8*(r/4) + 4*nt + r%4 for row r
    f32x4 sacc[2];
    long long krow[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
        krow[nt] = kv_row(kv, b, g, row_of(min(kb + 8 * (c16 >> 2) + 4 * nt + (c16 & 3), c_end - 1)));
    uint4 kraw[2][KPERM ? NQ / 2 : 1];
    uint32_t kscl[2][KPERM ? NQ / 2 : 1];
    if (KPERM) {  // all K codes and scales of the tile first
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int hh = 0; hh < NQ / 2; ++hh) {
                kraw[nt][hh] = *(const uint4*)((const int8_t*)kv.base[0] + krow[nt] * HD + 64 * hh + 16 * kgrp);
                kscl[nt][hh] = kv.base_scale[0][krow[nt] * NQ + 2 * hh + (kgrp >> 1)];
            }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const long long row = krow[nt];
        sacc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (KPERM) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const uint4 c4 = kraw[nt][j >> 1];
                const uint2 c = (j & 1) ? make_uint2(c4.z, c4.w) : make_uint2(c4.x, c4.y);
                const uint32_t sp = kscl[nt][j >> 1] | (kscl[nt][j >> 1] << 16);
                const uint4 kf = i8x8_to_f16(c, make_uint4(sp, sp, sp, sp));
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kf), as_half8(qop[j]), sacc[nt], 0, 0, 0);
            }
        } else if (I8) {
            const u16* ks = kv.base_scale[0] + row * NQ;
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const uint2 c = *(const uint2*)((const int8_t*)kv.base[0] + row * HD + 32 * j + 8 * kgrp);
                const uint32_t s1 = ks[j];
                const uint32_t sp = s1 | (s1 << 16);
                const uint4 kf = i8x8_to_f16(c, make_uint4(sp, sp, sp, sp));
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kf), as_half8(qop[j]), sacc[nt], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const uint4 kf = *(const uint4*)((const u16*)kv.base[0] + row * HD + 32 * j + 8 * kgrp);
                if (HALF)
                    sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kf), as_half8(qop[j]), sacc[nt], 0, 0, 0);
                else
                    sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qop[j]), sacc[nt], 0, 0, 0);
            }
        }
    }
    // lane (kgrp, head c16) holds keys kb + 8kgrp + 4nt + i
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kb + 8 * kgrp + 4 * nt + i;
            const float v = (key >= c_lo && key < c_end) ? sacc[nt][i] * sl2 : -INFINITY;
            s[nt * 4 + i] = v;
            mx = fmaxf(mx, v);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    float p[8];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = (s[j] == -INFINITY) ? 0.f : exp2f(s[j] - m_new);
        rs += p[j];
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int et = 0; et < NE; ++et) oacc[et] *= alpha;
    // ---- O^T += V^T P^T; lane (e, kgrp): V[keys kb+8kgrp .. +8][e] is one contiguous run
    uint4 pu;
    if (HALF) {
        pu.x = pack_h2(p[0], p[1]);
        pu.y = pack_h2(p[2], p[3]);
        pu.z = pack_h2(p[4], p[5]);
        pu.w = pack_h2(p[6], p[7]);
    } else {
        pu.x = pack_bf2(p[0], p[1]);
        pu.y = pack_bf2(p[2], p[3]);
        pu.z = pack_bf2(p[4], p[5]);
        pu.w = pack_bf2(p[6], p[7]);
    }
    const int valid = c_end - (kb + 8 * kgrp);
    // rows past the end of the context are unwritten: clamp the block address, zero the values
#pragma unroll
    for (int et = 0; et < NE; ++et) {
        uint4 vf;
        if (I8) {
            const uint4 c4 = vraw[et >> 1];
            const uint2 c = (et & 1) ? make_uint2(c4.z, c4.w) : make_uint2(c4.x, c4.y);
            vf = i8x8_to_f16(c, vsc[et >> 1]);
        } else {
            vf = vraw[et];
        }
        vf = mask_tail8(vf, valid);
        if (HALF)
            oacc[et] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(vf), as_half8(pu), oacc[et], 0, 0, 0);
        else
            oacc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), as_bf16x8(pu), oacc[et], 0, 0, 0);
    }
}

// Q^T operand of the decode attention for lane (kgrp, head c16) of KV head g of sequence
// b: q rotated here from the float32 projections (fuse_kv; one rounding to the
// operand type) or read from a.q (bf16, or float16 bits when q_half).
template <int HD, int G, int RT>
__device__ __forceinline__ void decode_q(const RowsAttn& a, int b, int g, int c16, int kgrp, uint4 (&qop)[HD / 32]) {
    constexpr bool I8 = RT == RT_I8;
    constexpr bool HALF = RT != RT_BF16;
    constexpr int NQ = HD / 32;
    const int Hkv = a.kv.Hkv;
    // int8 rows (hd >= 64): lane (key, kgrp) reads 16 bytes at 64h + 16 kgrp of its K row
    // for h < NQ / 2, so every load covers 64 contiguous bytes of each key; k-step j
    // takes elements 64 (j/2) + 16 kgrp + 8 (j%2) .. +8.  Other rows: 32 j + 8 kgrp.
    constexpr bool KPERM = I8 && NQ % 2 == 0;
    auto kslice = [&](int j) { return KPERM ? 64 * (j >> 1) + 16 * kgrp + 8 * (j & 1) : 32 * j + 8 * kgrp; };
    // Q^T operand: lane (head c16, kgrp) holds q[h][kslice(j) .. +8]
    const bool hvalid = c16 < G;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hvalid && a.fuse_kv) {  // rotate the float32 projection here
            // the 8 elements e0.. are pairs i0.. (one half of the head): 16-byte loads
            const int e0 = kslice(j), i0 = e0 % (HD / 2);
            const float* qh = a.qkv + (long long)b * (a.H + 2 * Hkv) * HD + (g * G + c16) * HD;
            float x1[8], x2[8], cs[16];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                *(float4*)&x1[4 * t] = *(const float4*)(qh + i0 + 4 * t);
                *(float4*)&x2[4 * t] = *(const float4*)(qh + i0 + HD / 2 + 4 * t);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) *(float4*)&cs[4 * t] = *(const float4*)(a.rope_cs + 2 * i0 + 4 * t);
            const bool lo = e0 < HD / 2;
            uint32_t o[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float r2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int m = 2 * t + u;
                    const float c = cs[2 * m], sn = cs[2 * m + 1];
                    r2[u] = lo ? rope_lo(x1[m], x2[m], c, sn) : rope_hi(x1[m], x2[m], c, sn);
                }
                // the float16 kernels take the rotated float32 q with one rounding
                o[t] = HALF ? (pack_h2(r2[0], r2[1])) : pack_bf2(r2[0], r2[1]);
            }
            v = make_uint4(o[0], o[1], o[2], o[3]);
        } else if (hvalid) {
            v = *(const uint4*)(a.q + (long long)b * a.H * HD + (g * G + c16) * HD + kslice(j));
        }
        if (HALF && !a.fuse_kv && !a.q_half) {  // bf16 -> f16
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                o[t] = pack_h2(__uint_as_float(wv[t] << 16), __uint_as_float(wv[t] & 0xFFFF0000u));
            v = make_uint4(o[0], o[1], o[2], o[3]);
        }
        qop[j] = v;
    }
}

// The int8 row type streams the loop-1 base from HBM and wants three waves per SIMD in
// flight; its register count sits just above that limit unless the bound asks for it.
template <int HD, int G, int RT>
__global__ __launch_bounds__(256, RT == RT_I8 || RT == RT_F16_2SEG || RT == RT_F16_2SEG_LIVE ? 3 : 1) void attn_decode_dense_kernel(RowsAttn a) {
    constexpr bool I8 = RT == RT_I8;
    constexpr bool HALF = RT != RT_BF16;  // f16 MFMA (int8 codes are converted to f16)
    constexpr bool SEG = RT == RT_F16_2SEG || RT == RT_F16_2SEG_LIVE;
    constexpr bool LIVE = RT == RT_F16_2SEG_LIVE;
    constexpr int NQ = HD / 32;   // 32-wide k-steps over hd (= scale groups)
    constexpr int NE = HD / 16;   // 16-row tiles of O^T
    const int split = blockIdx.x, bg = blockIdx.y;
    const bool seg2 = SEG && split >= a.seg_split;
    const KVLayer& kv = seg2 ? a.kv2 : a.kv;
    const int Hkv = kv.Hkv, b = bg / Hkv, g = bg % Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c16 = lane & 15, kgrp = lane >> 4;
    const float sl2 = kLog2e / sqrtf((float)HD);
    // Two segments, new-key split on: this workgroup writes the new token's K/V row and
    // forms that one key's partial from the values it wrote, with no load after the
    // write: thread (kv, e) holds K or V element e as the ring stores it (float16), the
    // K threads also the G float16 queries at e.  Score s_h = sum_e q_h[e] k[e] in
    // float32, weight exp2(0) = 1, output the V row.
    if (SEG && a.nk_split > 0 && split == a.nk_split) {
        const int pos = *a.dpos;
        const int kvh = threadIdx.x >> 7, e = threadIdx.x & 127;
        float val = 0.f, qf[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) qf[hh] = 0.f;
        if (e < HD) {
            const int i = e % (HD / 2);
            const float c = kvh == 0 ? a.rope_cs[2 * i] : 1.f;
            const float sn = kvh == 0 ? a.rope_cs[2 * i + 1] : 0.f;
            const float* src = a.qkv + (long long)b * (a.H + 2 * Hkv) * HD;
            if (kvh == 0) {  // the queries of the group's heads, rotated and rounded as decode_q does
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float* qh = src + (g * G + hh) * HD;
                    const float r = e < HD / 2 ? rope_lo(qh[i], qh[i + HD / 2], c, sn) : rope_hi(qh[i], qh[i + HD / 2], c, sn);
                    // a rotated q outside the float16 range raises the store's range flag
                    // (this workgroup rotates every q element of its group, once)
                    if (a.kvw.range_flag && !(fabsf(r) <= 65504.f)) *a.kvw.range_flag = 1u;
                    qf[hh] = h2f(f2h_bits(r));
                }
            }
            val = h2f(f2h_bits(kv_write_elem(src, a.H, Hkv, HD, b, g, kvh, e, pos, 0, c, sn, a.kvw,
                                             kvh == 0 && g == 0 && e == 0)));
        }
        if (LIVE && *a.live == 0) return;  // no sequence left in the loops: the write only
        __shared__ float sm_s[2][G];
        if (kvh == 0) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float t = wave_sum(qf[hh] * val);
                if (lane == 0) sm_s[w][hh] = t;
            }
        }
        __syncthreads();
        float* P = a.part + ((long long)bg * a.n_splits + split) * G * (HD + 2);
        if (kvh == 1 && e < HD) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) P[hh * (HD + 2) + e] = val;
        }
        if (threadIdx.x < G) {
            P[threadIdx.x * (HD + 2) + HD] = (sm_s[0][threadIdx.x] + sm_s[1][threadIdx.x]) * sl2;
            P[threadIdx.x * (HD + 2) + HD + 1] = 1.f;
        }
        return;
    }
    // S rows: the column of each thread's entry is loaded before the query, so that the
    // two loads are in flight together
    int s_col = 0x7fffffff;
    if (SEG && !seg2) {
        const int i = split * a.chunk + threadIdx.x;
        if (threadIdx.x < a.chunk && i < a.n_cols) s_col = a.cols[(long long)bg * a.n_cols + i];
    }
    // the new token's K/V row goes to the store first when this workgroup reads it
    // (without a new-key split)
    if (a.fuse_kv && a.nk_split == 0 && (!SEG || seg2)) {
        const int pos = *a.dpos;
        const int ring0 = SEG ? max(0, pos - a.window + 1) & ~7 : 0;
        const int key = pos - ring0;
        const int cb = (SEG ? split - a.seg_split : split) * a.chunk;
        if (key >= cb && key < cb + a.chunk) {
            const int kvh = threadIdx.x >> 7, e = threadIdx.x & 127;
            if (e < HD) {
                const float c = kvh == 0 ? a.rope_cs[2 * (e % (HD / 2))] : 1.f;
                const float sn = kvh == 0 ? a.rope_cs[2 * (e % (HD / 2)) + 1] : 0.f;
                kv_write_elem(a.qkv + (long long)b * (a.H + 2 * Hkv) * HD, a.H, Hkv, HD, b, g, kvh, e, pos, 0, c, sn,
                              a.kvw, kvh == 0 && g == 0 && e == 0);
            }
            __syncthreads();
        }
    }
    if (LIVE && *a.live == 0) return;  // no sequence left in the loops: the write only

    uint4 qop[NQ];
    decode_q<HD, G, RT>(a, b, g, c16, kgrp, qop);
    // keys [c_lo, c_end) of rows [c_begin, c_begin + chunk) take part
    int c_begin, c_lo, c_end, ring0 = 0;
    if (!SEG) {
        const int ncols = a.lens ? a.lens[bg] : (a.dpos ? *a.dpos : a.pos) + 1;
        c_begin = c_lo = split * a.chunk;
        c_end = min(ncols, c_begin + a.chunk);
    } else if (!seg2) {  // S rows: the ascending columns up to pos - window form a prefix
        const int pos = a.dpos ? *a.dpos : a.pos;
        __shared__ int s_cnt[4];
        c_begin = c_lo = split * a.chunk;
        const unsigned long long bal = __ballot(s_col <= pos - a.window);
        if (lane == 0) s_cnt[w] = __popcll(bal);
        __syncthreads();
        c_end = c_begin + s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    } else {  // window keys start at the 8-aligned position below the window
        const int pos = a.dpos ? *a.dpos : a.pos;
        const int wlo = max(0, pos - a.window + 1);
        ring0 = wlo & ~7;
        c_begin = (split - a.seg_split) * a.chunk;
        c_lo = max(c_begin, wlo - ring0);
        // with a new-key split, the new key (the last window key) is that split's
        c_end = min(c_begin + a.chunk, pos - ring0 + (a.nk_split > 0 ? 0 : 1));
    }
    // row of key `key` in kv (window ring: position ring0 + key at row % Tmax)
    auto row_of = [&](int key) { return seg2 ? (ring0 + key) % kv.Tmax : key; };
    const bool hvalid = c16 < G;
    f32x4 oacc[NE];
#pragma unroll
    for (int et = 0; et < NE; ++et) oacc[et] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (int kb = c_begin + 32 * w; kb < c_end; kb += 128)
        decode_tile<HD, G, RT>(kv, b, g, kb, c_lo, c_end, row_of, qop, oacc, m, l, sl2, c16, kgrp);
    // ---- merge the four waves: O^T lane holds row r = 4kgrp + i of tile et for head c16
    //      (head dim 16et + r; int8 rows: 32 (et/2) + 2r + et%2)
    __shared__ float sm_m[4][16], sm_l[4][16];
    __shared__ float sm_o[4][G][HD];
    if (kgrp == 0) {
        sm_m[w][c16] = m;
        sm_l[w][c16] = l;
    }
    if (hvalid) {
#pragma unroll
        for (int et = 0; et < NE; ++et)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * kgrp + i;
                sm_o[w][c16][I8 ? 32 * (et >> 1) + 2 * r + (et & 1) : 16 * et + r] = oacc[et][i];
            }
    }
    __syncthreads();
    float* P = a.part + ((long long)bg * a.n_splits + split) * G * (HD + 2);
    for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
        const int hh = idx / HD, e = idx % HD;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][hh]);
        float L = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                if (sm_m[ww][hh] == -INFINITY) continue;
                const float f = exp2f(sm_m[ww][hh] - M);
                L += f * sm_l[ww][hh];
                acc += f * sm_o[ww][hh][e];
            }
        }
        P[hh * (HD + 2) + e] = acc;
        if (e == 0) {
            P[hh * (HD + 2) + HD] = M;
            P[hh * (HD + 2) + HD + 1] = L;
        }
    }
}

// ---------------------------------------------------------------- sparse decode: gather
// 8 consecutive elements [e0, e0+8) of residual row rr (loop kk): added to x, or
// substituted for 16-bit residual rows.
template <int HD>
__device__ __forceinline__ void res8_apply(const KVLayer& v, int kv, int kk, long long rr, int e0, float* x) {
    if (v.res_bits == 16) {
        const uint4 u = *(const uint4*)((const u16*)v.res[kk - 2][kv] + rr * HD + e0);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w4[j] << 16);
            x[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
        }
        return;
    }
    const float s = h2f(v.res_scale[kk - 2][kv][rr * (HD / 32) + e0 / 32]);
    if (v.res_bits == 8) {
        const uint2 u = *(const uint2*)((const int8_t*)v.res[kk - 2][kv] + rr * HD + e0);
        const uint32_t w2[2] = {u.x, u.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = x[j] + (float)(int8_t)((w2[j >> 2] >> (8 * (j & 3))) & 0xFF) * s;
    } else {
        const uint32_t u = *(const uint32_t*)((const uint8_t*)v.res[kk - 2][kv] + rr * (HD / 2) + e0 / 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int nib = (int)((u >> (4 * j)) & 0xF);
            nib = nib >= 8 ? nib - 16 : nib;
            x[j] = x[j] + (float)nib * s;
        }
    }
}

// Block = 64 consecutive entries of one (b, g) column list.  The entries' positions
// and loop-2..k slots are staged in LDS.  K: 4 threads per entry, row-major, one
// contiguous run of hd/4 elements each.  V: 32 threads per 8 consecutive entries,
// each owning hd/32 head dims; when the 8 entries are 8 consecutive positions
// starting at a multiple of 8 (window, runs of S) the 8 keys of a head dim are one
// vector load from the 8-key-interleaved store.
template <int HD>
__global__ __launch_bounds__(256) void gather_recon_kernel(RowsAttn a, int mode, int ncap, u16* __restrict__ kc,
                                                           u16* __restrict__ vc) {
    constexpr int NCOL = 64;
    constexpr int TPC = 256 / NCOL;        // threads per entry for K
    constexpr int EPT = HD / TPC;          // K elements per thread (multiple of 8)
    constexpr int TPG = 256 / (NCOL / 8);  // threads per group of 8 entries for V
    constexpr int EPV = HD / TPG;          // V head dims per thread
    __shared__ int s_col[NCOL];
    __shared__ int s_slot[LK_MAX_LOOPS][NCOL];
    const KVLayer& v = a.kv;
    const int t = threadIdx.x;
    const int bg = blockIdx.y, Hkv = v.Hkv, b = bg / Hkv, g = bg % Hkv;
    const int32_t* S = a.cols ? a.cols + (long long)bg * a.n_cols : nullptr;
    const bool ring = mode == GATHER_RING;
    int cntS, ncols, win_lo;
    if (!ring) {
        cntS = ncols = a.n_cols;
        win_lo = 0;
    } else {
        const int T = (a.dpos ? *a.dpos : a.pos) + 1;
        cntS = 0;
        win_lo = (max(0, T - ncap) + 7) & ~7;
        ncols = T - win_lo;
    }
    // destination row of entry c (ring rows keep 8-aligned groups contiguous)
    auto dst_row = [&](int c) { return ring ? (win_lo + c) % ncap : c; };
    const int c0 = blockIdx.x * NCOL;
    const int nres = v.lazy ? a.k_loop - 1 : 0;
    if (t < NCOL) {
        const int c = c0 + t;
        int col = -1;
        if (c < ncols) col = c < cntS ? S[c] : win_lo + (c - cntS);
        s_col[t] = col;
        for (int kk = 0; kk < nres; ++kk)
            s_slot[kk][t] = col >= 0 ? v.slot[((long long)kk * v.B + b) * v.Tmax + col] : -1;
    }
    __syncthreads();
    {   // ---- K rows
        const int i = t / TPC, e0 = (t % TPC) * EPT;
        const int col = s_col[i];
        float x[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) x[j] = 0.f;
        if (col >= 0) {
            const long long row = kv_row(v, b, g, col);
#pragma unroll
            for (int j8 = 0; j8 < EPT / 8; ++j8) {
                const int e = e0 + 8 * j8;
                if (!v.lazy || v.base_bits == 16) {
                    const uint4 u = *(const uint4*)((const u16*)v.base[0] + row * HD + e);
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        x[8 * j8 + 2 * q] = __uint_as_float(w4[q] << 16);
                        x[8 * j8 + 2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
                    }
                } else {
                    const uint2 u = *(const uint2*)((const int8_t*)v.base[0] + row * HD + e);
                    const float sc = h2f(v.base_scale[0][row * (HD / 32) + e / 32]);
                    const uint32_t w2[2] = {u.x, u.y};
#pragma unroll
                    for (int q = 0; q < 8; ++q) x[8 * j8 + q] = (float)(int8_t)((w2[q >> 2] >> (8 * (q & 3))) & 0xFF) * sc;
                }
            }
            for (int kk = 2; kk <= nres + 1; ++kk) {
                const int sl = s_slot[kk - 2][i];
                if (sl < 0) continue;
                const long long rr = res_row(v, b, g, sl);
#pragma unroll
                for (int j8 = 0; j8 < EPT / 8; ++j8) res8_apply<HD>(v, 0, kk, rr, e0 + 8 * j8, x + 8 * j8);
            }
        }
        u16* dst = kc + ((long long)bg * ncap + dst_row(c0 + i)) * HD + e0;
#pragma unroll
        for (int j8 = 0; j8 < EPT / 8; ++j8) {
            if (ring && c0 + i >= ncols) break;
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_h2(x[8 * j8 + 2 * q], x[8 * j8 + 2 * q + 1]);
            *(uint4*)(dst + 8 * j8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    {   // ---- V, 8 entries at a time, written 8-key interleaved
        const int grp = t / TPG, e0 = (t % TPG) * EPV;
        const int cb = grp * 8;
        const int p0 = s_col[cb];
        bool run = p0 >= 0 && (p0 & 7) == 0;
#pragma unroll
        for (int j = 1; j < 8; ++j) run = run && s_col[cb + j] == p0 + j;
        float vx[8][EPV];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < EPV; ++q) vx[j][q] = 0.f;
        if (run) {
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
                const int e = e0 + q;
                const long long vi = v_elem(v, b, g, p0, e);
                if (!v.lazy || v.base_bits == 16) {
                    const uint4 u = *(const uint4*)((const u16*)v.base[1] + vi);
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        vx[2 * j][q] = __uint_as_float(w4[j] << 16);
                        vx[2 * j + 1][q] = __uint_as_float(w4[j] & 0xFFFF0000u);
                    }
                } else {
                    const uint2 u = *(const uint2*)((const int8_t*)v.base[1] + vi);
                    const u16* sp = v.base_scale[1] + v_scale_idx(v, b, g, p0, e / 32);
                    const uint32_t w2[2] = {u.x, u.y};
#pragma unroll
                    for (int j = 0; j < 8; ++j) vx[j][q] = (float)(int8_t)((w2[j >> 2] >> (8 * (j & 3))) & 0xFF) * h2f(sp[j]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = s_col[cb + j];
                if (col < 0) continue;
#pragma unroll
                for (int q = 0; q < EPV; ++q) vx[j][q] = kv_base_elem(v, 1, b, g, col, e0 + q);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s_col[cb + j] < 0) continue;
            for (int kk = 2; kk <= nres + 1; ++kk) {
                const int sl = s_slot[kk - 2][cb + j];
                if (sl < 0) continue;
#pragma unroll
                for (int q = 0; q < EPV; ++q) vx[j][q] = kv_apply_res(v, 1, b, g, kk, sl, e0 + q, vx[j][q]);
            }
        }
        const long long blk = (long long)bg * (ncap / 8) + dst_row(c0 + cb) / 8;
#pragma unroll
        for (int q = 0; q < EPV; ++q) {
            if (ring && c0 + cb >= ncols) break;
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_h2(vx[2 * j][q], vx[2 * j + 1][q]);
            *(uint4*)(vc + (blk * HD + e0 + q) * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// ---------------------------------------------------------------- sparse prefill rows (MFMA)
// Token-sparse prefill at loop k >= 2 for hd 128: kept query i attends over
// (S ∩ [0, i-w]) ∪ [i-w+1, i], the first part read from the float16 stable-column cache
// sc (row r = column cols[r]), the second from a float16 copy fr of the loop-k
// reconstruction at every prompt position.  A workgroup takes RB consecutive kept rows of
// one sequence for all G query heads of KV head g (wave w: head w % G, rows 32 (w / G) ..),
// so every K/V tile is read once for the G heads.  Tiles: first the cache rows with a
// column at or below (last row's position - w), then the positions from the first row's
// window start to the last row's position; per query both are masked exactly.  f16 MFMAs
// (q converted from bf16: exact for magnitudes in [2^-14, 65504]), online softmax as in the flash prefill, output written
// directly (no split partials).
template <int G>
__global__ __launch_bounds__(G > 4 ? 64 * G : 256, 2) void attn_rows_pf_kernel(RowsAttn a, KVLayer sc, KVLayer fr,
                                                                            float sl2) {
    constexpr int HD = 128, KT = 64, LDK = HD + 8, LDV = KT + 8, CPR = HD / 8;
    constexpr int NW = G > 4 ? G : 4, NT = NW * 64;
    constexpr int RB = 32 * NW / G;
    constexpr int NKC = KT * CPR, NVC = (KT / 8) * HD;
    constexpr int PER = (NKC + NVC) / NT;
    __shared__ __attribute__((aligned(16))) u16 Ks[2][KT * LDK];
    __shared__ __attribute__((aligned(16))) u16 Vt[2][HD * LDV];
    __shared__ int s_col[2][KT];
    __shared__ int s_pos[RB];
    __shared__ int s_cnt[NW];
    // wave index through readfirstlane: the per-wave tests are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, l32 = lane & 31;
    const int g = blockIdx.y, b = blockIdx.z, Hkv = a.kv.Hkv, H = a.H;
    const int bg = b * Hkv + g, n = a.n_rows, W = a.window;
    const int j0 = (gridDim.x - 1 - blockIdx.x) * RB;
    const int hh = w % G, rs = w / G, h = g * G + hh;
    for (int i = tid; i < RB; i += NT) s_pos[i] = j0 + i < n ? a.qpos[(long long)b * n + j0 + i] : -1;
    __syncthreads();
    const int jl = min(j0 + RB, n) - 1;
    const int Pf = __builtin_amdgcn_readfirstlane(s_pos[0]), Pl = __builtin_amdgcn_readfirstlane(s_pos[jl - j0]);
    const int32_t* S = a.cols + (long long)bg * a.n_cols;
    // columns at or below Pl - W (S ascending): counted by every thread over a stride,
    // one round of loads instead of a binary search's chain
    {
        int c = 0;
        for (int i = tid; i < a.n_cols; i += NT) c += S[i] <= Pl - W;
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
        if (lane == 0) s_cnt[w] = c;
    }
    __syncthreads();
    int cnt1 = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) cnt1 += s_cnt[i];
    cnt1 = __builtin_amdgcn_readfirstlane(cnt1);
    const int nt1 = (cnt1 + KT - 1) / KT;
    const int lo2 = max(0, Pf - W + 1) & ~7;
    const int ntiles = nt1 + (Pl - lo2) / KT + 1;
    const int jr = j0 + rs * 32 + l32;
    const int P = jr < n ? s_pos[rs * 32 + l32] : -1;
    const bool wave_rows = j0 + rs * 32 < n;
    const int wPf = __builtin_amdgcn_readfirstlane(wave_rows ? s_pos[rs * 32] : 0);
    const int wPl = __builtin_amdgcn_readfirstlane(wave_rows ? s_pos[min(j0 + rs * 32 + 31, n - 1) - j0] : -1);
    const long long ldq = (long long)H * HD;

    half8 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (jr < n) v = *(const uint4*)(a.q + ((long long)b * n + jr) * ldq + h * HD + ks * 16 + kg * 8);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        half8 hq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hq[2 * q] = (_Float16)__uint_as_float(wv[q] << 16);
            hq[2 * q + 1] = (_Float16)__uint_as_float(wv[q] & 0xFFFF0000u);
        }
        qf[ks] = hq;
    }
    f32x16 oacc[HD / 32];
#pragma unroll
    for (int c = 0; c < HD / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] = 0.f;
    float m_i = -INFINITY, l_i = 0.f;

    uint4 regs[PER];
    int colr = INT_MAX;  // tile column of key tid (seg 1), staged like the operands
    // A tile whose 64 keys all exist loads from fixed per-thread offsets (as the flash
    // prefill): K chunk p holds key k0 + (NT/16) p of the tile, V chunk p the 8 keys of
    // block tid/128 + (NT/128) (p - PK) at head dim tid % 128.
    constexpr int PK = NKC / NT;
    const int k0 = flash_key_of_row(tid / CPR);
    const int koff = k0 * HD + (tid % CPR) * 8;
    const int voff = (tid / HD) * HD * 8 + (tid % HD) * 8;
    auto load_tile = [&](int t) {
        const bool seg1 = t < nt1;
        const int base = seg1 ? t * KT : lo2 + (t - nt1) * KT;
        const int lim = seg1 ? cnt1 : Pl + 1;  // keys (rows or positions) below lim exist
        const KVLayer& L = seg1 ? sc : fr;
        if (tid < KT) colr = (seg1 && base + tid < cnt1) ? S[base + tid] : INT_MAX;
        if (base + KT <= lim) {
            const long long r = (long long)bg * L.Tmax + base;
            const u16* kb = (const u16*)L.base[0] + r * HD;
            const u16* vb = (const u16*)L.base[1] + r * HD;
#pragma unroll
            for (int p = 0; p < PK; ++p) regs[p] = *(const uint4*)(kb + koff + p * (NT / 16) * HD);
#pragma unroll
            for (int p = 0; p < PER - PK; ++p) regs[PK + p] = *(const uint4*)(vb + voff + p * NT * 8);
            return;
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            regs[p] = make_uint4(0, 0, 0, 0);
            if (c < NKC) {
                const int r = c / CPR;
                const int key = base + (r & 32) + flash_key_of_row(r & 31);
                if (key < lim)
                    regs[p] = *(const uint4*)((const u16*)L.base[0] + kv_row(L, b, g, key) * HD + (c % CPR) * 8);
            } else {
                const int cc = c - NKC;
                const int blk = cc / HD, e = cc % HD;
                const int p0 = base + blk * 8;
                if (p0 < lim) regs[p] = mask_tail8(*(const uint4*)((const u16*)L.base[1] + v_elem(L, b, g, p0, e)), lim - p0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            if (c < NKC) {
                *(uint4*)&Ks[buf][(c / CPR) * LDK + (c % CPR) * 8] = regs[p];
            } else {
                const int cc = c - NKC;
                *(uint4*)&Vt[buf][(cc % HD) * LDV + (cc / HD) * 8] = regs[p];
            }
        }
        if (tid < KT) s_col[buf][tid] = colr;
    };
    load_tile(0);
    store_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);
        const bool seg1 = t < nt1;
        const int pb = seg1 ? 0 : lo2 + (t - nt1) * KT;
        // does any query of this wave see a key of the tile?
        const bool live = wave_rows && (seg1 ? s_col[cur][0] <= wPl - W : (pb <= wPl && pb + KT - 1 > wPf - W));
        if (live) {
            f32x16 sv[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[hf][i] = 0.f;
#pragma unroll
                for (int ks = 0; ks < HD / 16; ++ks) {
                    const half8 k8 = as_half8(*(const uint4*)&Ks[cur][(32 * hf + l32) * LDK + ks * 16 + kg * 8]);
                    sv[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k8, qf[ks], sv[hf], 0, 0, 0);
                }
            }
            // every key of the tile visible to every row of the wave: no per-score mask
            const bool full = seg1 ? s_col[cur][KT - 1] <= wPf - W : (pb > wPl - W && pb + KT - 1 <= wPf);
            float mx = -INFINITY;
            if (full) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[hf][i]);
            } else {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kx = 32 * hf + ((i < 8) ? 8 * kg + i : 16 + 8 * kg + (i - 8));
                        const bool ok = seg1 ? s_col[cur][kx] <= P - W : (pb + kx <= P && pb + kx > P - W);
                        if (!ok) sv[hf][i] = -INFINITY;
                        mx = fmaxf(mx, sv[hf][i]);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_i, mx * sl2);
            if (__builtin_amdgcn_ballot_w64(m_new > m_i)) {
                const float alpha = (m_i == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
                l_i *= alpha;
#pragma unroll
                for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
            }
            m_i = m_new;
            const float nm = (m_new == -INFINITY) ? 0.f : -m_new;
            float rs_ = 0.f;
            half8 pf[2][2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int hq = 0; hq < 2; ++hq) {
                    half8 pv;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float x = __builtin_amdgcn_exp2f(fmaf(sv[hf][8 * hq + i], sl2, nm));
                        rs_ += x;
                        pv[i] = (_Float16)x;
                    }
                    pf[hf][hq] = pv;
                }
            }
            rs_ += __shfl_xor(rs_, 32);
            l_i += rs_;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int c = 0; c < HD / 32; ++c) {
                    const u16* vrow = &Vt[cur][(c * 32 + l32) * LDV + 32 * hf];
                    const half8 va0 = as_half8(*(const uint4*)(vrow + 8 * kg));
                    const half8 va1 = as_half8(*(const uint4*)(vrow + 16 + 8 * kg));
                    oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va0, pf[hf][0], oacc[c], 0, 0, 0);
                    oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va1, pf[hf][1], oacc[c], 0, 0, 0);
                }
        }
        if (t + 1 < ntiles) store_tile(cur ^ 1);
    }
    if (jr < n && l_i > 0.f) {
        const float inv = 1.f / l_i;
        u16* orow = a.out + ((long long)b * n + jr) * ldq + h * HD;
        if (a.diff_mode == DIFF_NONE) {
#pragma unroll
            for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int e0 = c * 32 + 8 * i4 + 4 * kg;
                    uint2 v;
                    v.x = pack_bf2(oacc[c][i4 * 4 + 0] * inv, oacc[c][i4 * 4 + 1] * inv);
                    v.y = pack_bf2(oacc[c][i4 * 4 + 2] * inv, oacc[c][i4 * 4 + 3] * inv);
                    *(uint2*)(orow + e0) = v;
                }
        } else {
            // difference correction: the row's float16 D at its position P
            u16* drow = a.d16 + ((long long)b * a.d_rows + P) * ldq + h * HD;
            const bool add = a.diff_mode == DIFF_ADD16;
#pragma unroll
            for (int c = 0; c < HD / 32; ++c)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int e0 = c * 32 + 8 * i4 + 4 * kg;
                    const uint2 dv = *(const uint2*)(drow + e0);
                    const uint2 ov = add ? dv : *(const uint2*)(orow + e0);
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wd = j < 2 ? dv.x : dv.y, wo = j < 2 ? ov.x : ov.y;
                        const float o = oacc[c][i4 * 4 + j] * inv;
                        x[j] = add ? o + h2f((u16)(wd >> (16 * (j & 1))))
                                   : __uint_as_float((j & 1) ? (wo & 0xFFFF0000u) : (wo << 16)) - o;
                    }
                    uint2 v;
                    if (add) {
                        v.x = pack_bf2(x[0], x[1]);
                        v.y = pack_bf2(x[2], x[3]);
                        *(uint2*)(orow + e0) = v;
                    } else {
                        v.x = pack_h2(x[0], x[1]);
                        v.y = pack_h2(x[2], x[3]);
                        *(uint2*)(drow + e0) = v;
                    }
                }
        }
    }
}

// ---------------------------------------------------------------- sparse rows (VALU)
// 32 consecutive K elements [e0, e0+32) of row (b, g, pos) reconstructed at loop k,
// given that row's loop-2..k slots.
template <int HD>
__device__ __forceinline__ void recon_k32(const KVLayer& v, int b, int g, int pos, int e0, int k,
                                          const int* slots, float* x) {
    const long long row = kv_row(v, b, g, pos);
    if (!v.lazy || v.base_bits == 16) {
        const uint4* src = (const uint4*)((const u16*)v.base[0] + row * HD + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = src[q];
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[q * 8 + 2 * j] = __uint_as_float(w4[j] << 16);
                x[q * 8 + 2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float s = h2f(v.base_scale[0][row * (HD / 32) + e0 / 32]);
        const uint4* src = (const uint4*)((const int8_t*)v.base[0] + row * HD + e0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 u = src[q];
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) x[q * 16 + j * 4 + t] = (float)(int8_t)((w4[j] >> (8 * t)) & 0xFF) * s;
        }
    }
    if (!v.lazy) return;
    for (int kk = 2; kk <= k; ++kk) {
        const int sl = slots[kk - 2];
        if (sl < 0) continue;
        const long long rr = res_row(v, b, g, sl);
        if (v.res_bits == 16) {
            const uint4* src = (const uint4*)((const u16*)v.res[kk - 2][0] + rr * HD + e0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 u = src[q];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[q * 8 + 2 * j] = __uint_as_float(w4[j] << 16);
                    x[q * 8 + 2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
                }
            }
        } else {
            const float s = h2f(v.res_scale[kk - 2][0][rr * (HD / 32) + e0 / 32]);
            if (v.res_bits == 8) {
                const uint4* src = (const uint4*)((const int8_t*)v.res[kk - 2][0] + rr * HD + e0);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint4 u = src[q];
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            x[q * 16 + j * 4 + t] = x[q * 16 + j * 4 + t] +
                                                    (float)(int8_t)((w4[j] >> (8 * t)) & 0xFF) * s;
                }
            } else {
                const uint4 u = *(const uint4*)((const uint8_t*)v.res[kk - 2][0] + rr * (HD / 2) + e0 / 2);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        int nib = (int)((w4[j] >> (4 * t)) & 0xF);
                        nib = nib >= 8 ? nib - 16 : nib;
                        x[j * 8 + t] = x[j * 8 + t] + (float)nib * s;
                    }
            }
        }
    }
}

// V element e of column (b, g, pos) at loop k; slots[(kk-2) * 64] is the column's loop-kk slot.
__device__ __forceinline__ float recon_v(const KVLayer& v, int b, int g, int pos, int e, int k, const int* slots) {
    float x = kv_base_elem(v, 1, b, g, pos, e);
    if (!v.lazy) return x;
    for (int kk = 2; kk <= k; ++kk) {
        const int sl = slots[(kk - 2) * 64];
        if (sl >= 0) x = kv_apply_res(v, 1, b, g, kk, sl, e, x);
    }
    return x;
}

template <int HD, int G>
__global__ __launch_bounds__(64) void attn_rows_kernel(RowsAttn a) {
    constexpr int DPL = HD >= 64 ? HD / 64 : 1;   // head dims per lane in p.V
    const int row = blockIdx.x, split = blockIdx.y, bg = blockIdx.z;
    const int Hkv = a.kv.Hkv;
    const int b = bg / Hkv, g = bg % Hkv;
    const int lane = threadIdx.x;
    const long long qrow = (long long)b * a.n_rows + row;
    const int pos = a.qpos ? a.qpos[qrow] : (a.dpos ? *a.dpos : a.pos);
    const int nres = a.kv.lazy ? a.k_loop - 1 : 0;
    __shared__ float qs[G][HD];
    __shared__ float ps[G][64];
    __shared__ int cs[64];
    __shared__ int slot_s[LK_MAX_LOOPS][64];
    const float scale = kLog2e / sqrtf((float)HD);
    for (int idx = lane; idx < G * HD; idx += 64) {
        const int hh = idx / HD, e = idx % HD;
        qs[hh][e] = bf2f(a.q[qrow * a.H * HD + (g * G + hh) * HD + e]) * scale;
    }
    const int32_t* S = a.cols + ((long long)b * Hkv + g) * a.n_cols;
    const int lim = pos - a.window;  // S columns at or below lim lie outside the window
    int lo = 0, hi = a.n_cols;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (S[mid] <= lim) lo = mid + 1;
        else hi = mid;
    }
    const int cntS = lo;
    const int win_lo = max(0, pos - a.window + 1);
    const int ncols = cntS + (pos - win_lo + 1);
    const int c_begin = split * a.chunk;
    const int c_end = min(ncols, c_begin + a.chunk);
    float m[G], l[G], o[G][DPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) o[hh][dd] = 0.f;
    }
    __syncthreads();
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
        const int c = c0 + lane;
        const bool valid = c < c_end;
        const int col = valid ? (c < cntS ? S[c] : win_lo + (c - cntS)) : 0;
        int myslots[LK_MAX_LOOPS];
        for (int kk = 0; kk < nres; ++kk) {
            myslots[kk] = valid ? a.kv.slot[((long long)kk * a.kv.B + b) * a.kv.Tmax + col] : -1;
            slot_s[kk][lane] = myslots[kk];
        }
        float s[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
        if (valid) {
            for (int e0 = 0; e0 < HD; e0 += 32) {
                float x[32];
                recon_k32<HD>(a.kv, b, g, col, e0, a.k_loop, myslots, x);
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
#pragma unroll
                    for (int e = 0; e < 32; ++e) s[hh] += qs[hh][e0 + e] * x[e];
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float sv = valid ? s[hh] : -INFINITY;
            const float mx = wave_max(sv);
            const float m_new = fmaxf(m[hh], mx);
            const float alpha = (m[hh] == -INFINITY) ? 0.f : exp2f(m[hh] - m_new);
            const float p = valid ? exp2f(sv - m_new) : 0.f;
            l[hh] = l[hh] * alpha + wave_sum(p);
            m[hh] = m_new;
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) o[hh][dd] *= alpha;
            ps[hh][lane] = p;
        }
        cs[lane] = col;
        __syncthreads();
        const int cnt = min(64, c_end - c0);
        const int e = lane * DPL;
        if (e < HD) {
#pragma unroll 4
            for (int cc = 0; cc < cnt; ++cc) {
                const int colv = cs[cc];
                float vv[DPL];
#pragma unroll
                for (int dd = 0; dd < DPL; ++dd) vv[dd] = recon_v(a.kv, b, g, colv, e + dd, a.k_loop, &slot_s[0][cc]);
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float pp = ps[hh][cc];
#pragma unroll
                    for (int dd = 0; dd < DPL; ++dd) o[hh][dd] += pp * vv[dd];
                }
            }
        }
        __syncthreads();
    }
    float* P = a.part + ((qrow * Hkv + g) * a.n_splits + split) * (long long)G * (HD + 2);
    const int e = lane * DPL;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        if (e < HD)
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) P[hh * (HD + 2) + e + dd] = o[hh][dd];
        if (lane == 0) {
            P[hh * (HD + 2) + HD] = m[hh];
            P[hh * (HD + 2) + HD + 1] = l[hh];
        }
    }
}

// Split merge of the decode attention.  Splits that saw no key carry m = -inf and
// weigh 0.
constexpr int kCombineMaxSplits = 256, kCombineMaxG = 8;
// One block per (query row, query head), 128 threads.  Split s holds, for each of the G
// heads of its KV group, the unnormalised output o_s (hd floats) followed by its running
// max m_s (log2 units) and sum l_s.  Weights w_s = 2^(m_s - max m); out = sum w_s o_s /
// sum w_s l_s.  Every load of the first 32 splits (o_s[e] per thread and output dim,
// m_s and l_s per lane and split) is issued before any arithmetic, so a launch with up
// to 32 splits waits on one memory round trip.
constexpr int kCombinePre = 32;
// The difference correction of the merged rows (RowsAttn's diff_* fields).
struct DiffOut {
    int mode;
    float* d32;
    u16* d16;
    int d_rows, n_rows;
    const int32_t* qpos;
    const int32_t* live;
};
template <bool LIVE>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part, int n_splits, int G,
                                                           int HD, int H, int Hkv, u16* __restrict__ out,
                                                           bool packed, DiffOut df) {
    if (LIVE && *df.live == 0) return;  // no sequence left in the loops
    const long long qrow = blockIdx.x;
    const int head = blockIdx.y, g = head / G, hh = head % G;
    const int tid = threadIdx.x;
    const long long stride = (long long)G * (HD + 2);
    const float* ph = part + (qrow * Hkv + g) * (long long)n_splits * stride + hh * (HD + 2);
    const bool has_e = tid < HD;
    const float* pe = ph + (has_e ? tid : 0);
    const int lane = tid & 63;
    // Each wave forms the split weights by itself, with no exchange through LDS and no
    // barrier: lane l reads the (m, l) pairs of splits l, l + 64, ..., the wave reduces
    // the maximum and the weighted sum, and the weights of splits below 64 are read back
    // from their lanes.  The partial outputs of the thread's own element are loaded first.
    float v[kCombinePre];
#pragma unroll
    for (int u = 0; u < kCombinePre; ++u) v[u] = (has_e && u < n_splits) ? pe[u * stride] : 0.f;
    const float m_own = lane < n_splits ? ph[lane * stride + HD] : -INFINITY;
    const float l_own = lane < n_splits ? ph[lane * stride + HD + 1] : 0.f;
    float mloc = m_own;
    for (int s = lane + 64; s < n_splits; s += 64) mloc = fmaxf(mloc, ph[s * stride + HD]);
    const float M = wave_max(mloc);
    auto weight = [&](float m_s) { return (m_s == -INFINITY) ? 0.f : exp2f(m_s - M); };
    const float w_own = weight(m_own);
    float lloc = w_own * l_own;
    for (int s = lane + 64; s < n_splits; s += 64) lloc += weight(ph[s * stride + HD]) * ph[s * stride + HD + 1];
    const float inv = 1.0f / wave_sum(lloc);
    auto split_weight = [&](int s) {
        return s < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_own), s))
                      : weight(ph[s * stride + HD]);
    };
    for (int e = tid; e < HD; e += 128) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (e == tid) {
#pragma unroll
            for (int u = 0; u < kCombinePre; ++u)
                if (u < n_splits) acc[u & 3] += split_weight(u) * v[u];
            for (int s = kCombinePre; s < n_splits; ++s) acc[s & 3] += split_weight(s) * ph[s * stride + e];
        } else {
            for (int s = 0; s < n_splits; ++s) acc[s & 3] += split_weight(s) * ph[s * stride + e];
        }
        const float o = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * inv;
        const int k = head * HD + e;
        const long long oi = packed ? pk_index((int)qrow, k, H * HD) : qrow * H * HD + k;
        const long long di = qrow * H * HD + k;
        // packed (decode products): float16 in the lane-packed order
        auto put = [&](float y) { out[oi] = packed ? f2h_bits(y) : f2bf(y); };
        switch (df.mode) {
            case DIFF_ADD32: put(o + df.d32[di]); break;
            case DIFF_SET32:
                df.d32[di] = o;
                put(o);
                break;
            case DIFF_SUB32: df.d32[di] -= o; break;
            case DIFF_ADD16:
            case DIFF_OUT16: {
                const long long b = qrow / df.n_rows;
                const long long ri = (b * df.d_rows + df.qpos[qrow]) * H * HD + k;
                if (df.mode == DIFF_ADD16) out[oi] = f2bf(o + h2f(df.d16[ri]));
                else df.d16[ri] = f2h_bits(bf2f(out[oi]) - o);
                break;
            }
            default: put(o); break;
        }
    }
}

// waves per workgroup of the hd-128 flash prefill
constexpr int kFlashWaves = 8;

template <int HD>
hipError_t prefill_hd(const u16* q, const KVLayer& kv, int B, int T, int H, u16* out, float* lse,
                      hipStream_t st) {
    dim3 grid((T + 127) / 128, H, B);
    const float sl2 = kLog2e / sqrtf((float)HD);
    if (HD == 128) {
        constexpr int NW = kFlashWaves;
        dim3 fgrid((T + 32 * NW - 1) / (32 * NW), H, B);
        if (kv.lazy && kv.base_bits == 8)
            hipLaunchKernelGGL((attn_prefill_fa_kernel<true, NW>), fgrid, dim3(64 * NW), 0, st, q, kv, T, H, out, lse,
                               sl2);
        else
            hipLaunchKernelGGL((attn_prefill_fa_kernel<false, NW>), fgrid, dim3(64 * NW), 0, st, q, kv, T, H, out, lse,
                               sl2);
        return hipGetLastError();
    }
    if (kv.lazy && kv.base_bits == 8)
        hipLaunchKernelGGL((attn_prefill_kernel<HD, true>), grid, dim3(256), 0, st, q, kv, T, H, out, lse, sl2);
    else
        hipLaunchKernelGGL((attn_prefill_kernel<HD, false>), grid, dim3(256), 0, st, q, kv, T, H, out, lse, sl2);
    return hipGetLastError();
}

template <int HD>
hipError_t mass_hd(const u16* q, const KVLayer& kv, const float* lse, int B, int T, int H, float* mass,
                   hipStream_t st) {
    const float sl2 = kLog2e / sqrtf((float)HD);
    const bool i8 = kv.lazy && kv.base_bits == 8;
    if (T >= 4096) {  // long prompts: 256 keys per workgroup
        dim3 grid((T + 255) / 256, kv.Hkv, B);
        if (i8)
            hipLaunchKernelGGL((column_mass_kernel<HD, true, 8, 4>), grid, dim3(512), 0, st, q, kv, lse, T, H, mass, sl2);
        else
            hipLaunchKernelGGL((column_mass_kernel<HD, false, 8, 4>), grid, dim3(512), 0, st, q, kv, lse, T, H, mass, sl2);
        return hipGetLastError();
    }
    dim3 grid((T + 127) / 128, kv.Hkv, B);
    if (i8)
        hipLaunchKernelGGL((column_mass_kernel<HD, true, 4, 1>), grid, dim3(256), 0, st, q, kv, lse, T, H, mass, sl2);
    else
        hipLaunchKernelGGL((column_mass_kernel<HD, false, 4, 1>), grid, dim3(256), 0, st, q, kv, lse, T, H, mass, sl2);
    return hipGetLastError();
}

template <int HD, int G>
void dense_launch(const RowsAttn& a, hipStream_t st) {
    dim3 grid(a.n_splits, a.B * a.kv.Hkv);
    if (a.seg_split > 0 && a.live)
        hipLaunchKernelGGL((attn_decode_dense_kernel<HD, G, RT_F16_2SEG_LIVE>), grid, dim3(256), 0, st, a);
    else if (a.seg_split > 0)
        hipLaunchKernelGGL((attn_decode_dense_kernel<HD, G, RT_F16_2SEG>), grid, dim3(256), 0, st, a);
    else if (a.kv.lazy && a.kv.base_bits == 8)
        hipLaunchKernelGGL((attn_decode_dense_kernel<HD, G, RT_I8>), grid, dim3(256), 0, st, a);
    else if (!a.kv.lazy && a.kv.f16)
        hipLaunchKernelGGL((attn_decode_dense_kernel<HD, G, RT_F16>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((attn_decode_dense_kernel<HD, G, RT_BF16>), grid, dim3(256), 0, st, a);
}

template <int HD>
void dense_hd(const RowsAttn& a, int G, hipStream_t st) {
    switch (G) {
        case 1: dense_launch<HD, 1>(a, st); break;
        case 2: dense_launch<HD, 2>(a, st); break;
        case 4: dense_launch<HD, 4>(a, st); break;
        default: dense_launch<HD, 8>(a, st); break;
    }
}

template <int HD, int G>
void rows_launch(const RowsAttn& a, hipStream_t st) {
    dim3 grid(a.n_rows, a.n_splits, a.B * a.kv.Hkv);
    hipLaunchKernelGGL((attn_rows_kernel<HD, G>), grid, dim3(64), 0, st, a);
}

template <int HD>
void rows_hd(const RowsAttn& a, int G, hipStream_t st) {
    switch (G) {
        case 1: rows_launch<HD, 1>(a, st); break;
        case 2: rows_launch<HD, 2>(a, st); break;
        case 4: rows_launch<HD, 4>(a, st); break;
        default: rows_launch<HD, 8>(a, st); break;
    }
}

}  // namespace

hipError_t attn_prefill(const u16* q, const KVLayer& kv, int B, int T, int H, u16* out, float* lse,
                        hipStream_t st) {
    switch (kv.hd) {
        case 32: return prefill_hd<32>(q, kv, B, T, H, out, lse, st);
        case 64: return prefill_hd<64>(q, kv, B, T, H, out, lse, st);
        default: return prefill_hd<128>(q, kv, B, T, H, out, lse, st);
    }
}

hipError_t column_mass(const u16* q, const KVLayer& kv, const float* lse, int B, int T, int H,
                       float* mass, hipStream_t st) {
    switch (kv.hd) {
        case 32: return mass_hd<32>(q, kv, lse, B, T, H, mass, st);
        case 64: return mass_hd<64>(q, kv, lse, B, T, H, mass, st);
        default: return mass_hd<128>(q, kv, lse, B, T, H, mass, st);
    }
}

hipError_t attn_rows_main(const RowsAttn& a, hipStream_t st) {
    const int G = a.H / a.kv.Hkv;
    if (a.cols && a.seg_split == 0) {
        switch (a.kv.hd) {
            case 32: rows_hd<32>(a, G, st); break;
            case 64: rows_hd<64>(a, G, st); break;
            default: rows_hd<128>(a, G, st); break;
        }
    } else {
        switch (a.kv.hd) {
            case 32: dense_hd<32>(a, G, st); break;
            case 64: dense_hd<64>(a, G, st); break;
            default: dense_hd<128>(a, G, st); break;
        }
    }
    return hipGetLastError();
}

hipError_t attn_rows_prefill(const RowsAttn& a, const KVLayer& sc, const KVLayer& fr, hipStream_t st) {
    const int G = a.H / a.kv.Hkv;
    if (a.kv.hd != 128 || !a.cols || !a.qpos || a.n_rows < 1 || sc.Tmax % 8 || fr.Tmax % 8)
        return hipErrorInvalidValue;
    if (a.diff_mode != DIFF_NONE && ((a.diff_mode != DIFF_ADD16 && a.diff_mode != DIFF_OUT16) || !a.d16))
        return hipErrorInvalidValue;
    const int NW = G > 4 ? G : 4, RB = 32 * NW / G;
    dim3 grid((a.n_rows + RB - 1) / RB, a.kv.Hkv, a.B);
    const float sl2 = kLog2e / sqrtf(128.f);
    switch (G) {
        case 1: hipLaunchKernelGGL((attn_rows_pf_kernel<1>), grid, dim3(256), 0, st, a, sc, fr, sl2); break;
        case 2: hipLaunchKernelGGL((attn_rows_pf_kernel<2>), grid, dim3(256), 0, st, a, sc, fr, sl2); break;
        case 4: hipLaunchKernelGGL((attn_rows_pf_kernel<4>), grid, dim3(256), 0, st, a, sc, fr, sl2); break;
        case 8: hipLaunchKernelGGL((attn_rows_pf_kernel<8>), grid, dim3(512), 0, st, a, sc, fr, sl2); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t gather_recon(const RowsAttn& a, int mode, int ncap, u16* kc, u16* vc, hipStream_t st) {
    if (ncap % 64 || (mode != GATHER_ALL_S && mode != GATHER_RING)) return hipErrorInvalidValue;
    dim3 grid(ncap / 64, a.B * a.kv.Hkv);
    switch (a.kv.hd) {
        case 32: hipLaunchKernelGGL(gather_recon_kernel<32>, grid, dim3(256), 0, st, a, mode, ncap, kc, vc); break;
        case 64: hipLaunchKernelGGL(gather_recon_kernel<64>, grid, dim3(256), 0, st, a, mode, ncap, kc, vc); break;
        default: hipLaunchKernelGGL(gather_recon_kernel<128>, grid, dim3(256), 0, st, a, mode, ncap, kc, vc); break;
    }
    return hipGetLastError();
}

hipError_t attn_rows_combine(const RowsAttn& a, hipStream_t st, bool packed_out) {
    const int G = a.H / a.kv.Hkv;
    if (a.n_splits > kCombineMaxSplits || G > kCombineMaxG) return hipErrorInvalidValue;
    if (packed_out && (a.B * a.n_rows > 8 || (a.H * a.kv.hd) % 64)) return hipErrorInvalidValue;
    if ((a.diff_mode == DIFF_ADD32 || a.diff_mode == DIFF_SET32 || a.diff_mode == DIFF_SUB32) && !a.d32)
        return hipErrorInvalidValue;
    if ((a.diff_mode == DIFF_ADD16 || a.diff_mode == DIFF_OUT16) && (!a.d16 || !a.qpos || packed_out))
        return hipErrorInvalidValue;
    const DiffOut df{a.diff_mode, a.d32, a.d16, a.d_rows, a.n_rows, a.qpos, a.live};
    dim3 grid(a.B * a.n_rows, a.H);
    if (a.live)
        hipLaunchKernelGGL(attn_combine_kernel<true>, grid, dim3(128), 0, st, a.part, a.n_splits, G, a.kv.hd, a.H,
                           a.kv.Hkv, a.out, packed_out, df);
    else
        hipLaunchKernelGGL(attn_combine_kernel<false>, grid, dim3(128), 0, st, a.part, a.n_splits, G, a.kv.hd, a.H,
                           a.kv.Hkv, a.out, packed_out, df);
    return hipGetLastError();
}

}  // namespace lk
