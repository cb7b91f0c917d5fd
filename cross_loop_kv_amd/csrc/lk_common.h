// Device helpers shared by the gfx950 kernels of the looped-KV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LK_MAX_LOOPS 16
#define LK_WAVE 64

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf2f(u16 v) { return __uint_as_float((uint32_t)v << 16); }

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// Round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

// Two floats as packed bf16, a in the low half (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// Eight bf16 (16 bytes) reinterpreted as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- float16
__device__ __forceinline__ u16 f2h_bits(float f) {
    _Float16 h = (_Float16)f;  // IEEE round to nearest even
    return __builtin_bit_cast(u16, h);
}
__device__ __forceinline__ float h2f(u16 bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}
// Two floats as packed float16, a in the low half, round to nearest even (one
// v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, f16x2v));
}

// ---------------------------------------------------------------- rotary embedding
// Rotate-half RoPE of the pair (x1, x2) = (x[i], x[i + hd/2]) by an angle with cosine c
// and sine sn: x1' = x1 c - x2 sn, x2' = x2 c + x1 sn.  Each product is rounded before
// the sum (no fused multiply-add), so the rotated value is the same float32 as the
// plain elementwise evaluation of the formula.
__device__ __forceinline__ float rope_lo(float x1, float x2, float c, float sn) {
#pragma clang fp contract(off)
    return x1 * c - x2 * sn;
}
__device__ __forceinline__ float rope_hi(float x1, float x2, float c, float sn) {
#pragma clang fp contract(off)
    return x2 * c + x1 * sn;
}

// ---------------------------------------------------------------- reductions
// Butterfly reductions: every lane ends with the same, run-to-run identical value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Block-wide sum (blockDim.x multiple of 64, <= 1024); `red` holds >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

// ---------------------------------------------------------------- residual quantizer
// One group of 32 values held by 32 consecutive lanes (lane & 31 = element).
// scale = fp16_rne(min(amax / qmax, 65504)); code = 0 if scale == 0 else
// clamp(rint_half_even(r / scale), -qmax, qmax).  Divisions are IEEE float32.
__device__ __forceinline__ int quant_group32(float r, int qmax, u16* scale_bits) {
    float a = fabsf(r);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    float s32 = __fdiv_rn(a, (float)qmax);
    s32 = fminf(s32, 65504.f);
    u16 sb = f2h_bits(s32);
    float s = h2f(sb);
    *scale_bits = sb;
    if (s == 0.f) return 0;
    float c = rintf(__fdiv_rn(r, s));
    c = fminf(fmaxf(c, (float)-qmax), (float)qmax);
    return (int)c;
}

// ---------------------------------------------------------------- decode operand layout
// Decode products (at most 8 activation rows, K % 64 == 0) read their operands in a
// "lane-packed" order: for 8-row tile t and 32-element chunk c of each half of K,
// the 16-byte operand of MFMA lane l = 16 grp + 8 h + r (row 8t + r, elements
// h K/2 + 32 c + 8 grp .. +8) is stored at ((t * K/64 + c) * 64 + l) * 8, so every
// wave load is 1 KB contiguous.  Activations use tile 0 (rows < 8).
__host__ __device__ __forceinline__ long long pk_index(int row, int k, int K) {
    const int Kh = K >> 1, h = k >= Kh ? 1 : 0, kk = k - h * Kh;
    const long long tile = row >> 3;
    const int lane = ((kk >> 3) & 3) * 16 + h * 8 + (row & 7);
    return ((tile * (K >> 6) + (kk >> 5)) * 64 + lane) * 8 + (k & 7);
}

// ---------------------------------------------------------------- KV store views
// Address arithmetic of one shared layer of a lazy store (or a plain bf16 row
// cache when lazy == 0).  Positions are padded to Tmax (a multiple of 8).
//  * K rows: [b][g][pos][hd];  int8 K scales: [b][g][pos][hd/32].
//  * V rows: 8-key interleaved [b][g][pos/8][hd][8] (element (pos, e) at
//    ((b*Hkv + g)*Tmax/8 + pos/8)*hd*8 + e*8 + pos%8), so that the 8 keys of
//    one head dimension are contiguous -- the k-operand layout of the PV MFMA;
//    int8 V scales: [b][g][pos/8][hd/32][8].
//  * loop-k residual rows (K and V alike): [b][g][slot][row_bytes] with float16
//    scales [b][g][slot][hd/32].
struct KVLayer {
    int lazy;            // 0: plain rows in base[] (bf16, or f16 when f16 != 0); 1: lazy store
    int f16;             // plain rows hold float16 (a materialized reconstruction)
    int B, Hkv, hd, Tmax;
    long long slots;     // residual slots per (b, g)
    int base_bits;       // 16 or 8
    int res_bits;        // 16, 8 or 4
    int n_loops;         // K
    const void* base[2];          // [K|V]: bf16 rows or int8 codes
    const u16* base_scale[2];     // fp16 bits
    const void* res[LK_MAX_LOOPS][2];        // index kk-2 for loop kk
    const u16* res_scale[LK_MAX_LOOPS][2];
    const int32_t* slot;          // [K-1][B][Tmax]
};

__device__ __forceinline__ long long kv_row(const KVLayer& v, int b, int g, int pos) {
    return ((long long)(b * v.Hkv + g) * v.Tmax + pos);
}
__device__ __forceinline__ long long v_elem(const KVLayer& v, int b, int g, int pos, int e) {
    return ((((long long)(b * v.Hkv + g) * (v.Tmax >> 3) + (pos >> 3)) * v.hd + e) << 3) + (pos & 7);
}
__device__ __forceinline__ long long v_scale_idx(const KVLayer& v, int b, int g, int pos, int q) {
    return ((((long long)(b * v.Hkv + g) * (v.Tmax >> 3) + (pos >> 3)) * (v.hd >> 5) + q) << 3) + (pos & 7);
}
__device__ __forceinline__ long long res_row(const KVLayer& v, int b, int g, long long slot) {
    return ((long long)(b * v.Hkv + g) * v.slots + slot);
}
__device__ __forceinline__ int res_row_bytes(const KVLayer& v) {
    return v.res_bits == 16 ? v.hd * 2 : v.hd * v.res_bits / 8;
}

// Base (loop-1 / plain-row) value of element e of K (kv=0) or V (kv=1) at (b, g, pos).
__device__ __forceinline__ float kv_base_elem(const KVLayer& v, int kv, int b, int g, int pos, int e) {
    const long long idx = kv == 0 ? kv_row(v, b, g, pos) * v.hd + e : v_elem(v, b, g, pos, e);
    if (!v.lazy || v.base_bits == 16) return bf2f(((const u16*)v.base[kv])[idx]);
    const int8_t c = ((const int8_t*)v.base[kv])[idx];
    const long long si = kv == 0 ? kv_row(v, b, g, pos) * (v.hd / 32) + e / 32 : v_scale_idx(v, b, g, pos, e / 32);
    return (float)c * h2f(v.base_scale[kv][si]);
}

// Add (or, for 16-bit residuals, substitute) the loop-kk entry of element e.
__device__ __forceinline__ float kv_apply_res(const KVLayer& v, int kv, int b, int g, int kk, int sl, int e,
                                              float x) {
    const long long rr = res_row(v, b, g, sl);
    if (v.res_bits == 16) return bf2f(((const u16*)v.res[kk - 2][kv])[rr * v.hd + e]);
    int c;
    if (v.res_bits == 8) {
        c = ((const int8_t*)v.res[kk - 2][kv])[rr * v.hd + e];
    } else {
        const uint8_t byte = ((const uint8_t*)v.res[kk - 2][kv])[rr * (v.hd / 2) + e / 2];
        const int nib = (e & 1) ? (byte >> 4) : (byte & 0xF);
        c = nib >= 8 ? nib - 16 : nib;
    }
    return x + (float)c * h2f(v.res_scale[kk - 2][kv][rr * (v.hd / 32) + e / 32]);
}

// Value of element e of row (b, g, pos) reconstructed at loop `k`: base, then the
// loop 2..k residuals (16-bit residual rows replace).
__device__ __forceinline__ float kv_recon_elem(const KVLayer& v, int kv, int b, int g, int pos, int e, int k) {
    float x = kv_base_elem(v, kv, b, g, pos, e);
    if (!v.lazy) return x;
    for (int kk = 2; kk <= k; ++kk) {
        const int sl = v.slot[((long long)(kk - 2) * v.B + b) * v.Tmax + pos];
        if (sl >= 0) x = kv_apply_res(v, kv, b, g, kk, sl, e, x);
    }
    return x;
}
