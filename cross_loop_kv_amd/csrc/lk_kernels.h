// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher enqueues on `st` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lk_common.h"

namespace lk {

// ---- elementwise / selection (k_elem.hip)
// h[r] = tok_emb[clamp(ids[r], 0, vocab-1)] as float32.
hipError_t embed(const int32_t* ids, const u16* tok_emb, float* h, int rows, int d, int vocab,
                 hipStream_t st);
// if add != nullptr: x += add (written back).  Then y = x / sqrt(mean(x^2) + eps) * gain,
// stored as bf16 (out_bf) or float32 (out_f32).
hipError_t rmsnorm(float* x, const u16* add, const u16* gain, float eps, int rows, int d,
                   u16* out_bf, float* out_f32, hipStream_t st);
hipError_t add_rows(float* x, const u16* add, int rows, int d, hipStream_t st);
hipError_t copy_f32(const float* src, float* dst, long long n, hipStream_t st);
hipError_t add_f32(float* x, const float* y, long long n, hipStream_t st);  // x += y
hipError_t fill_i32(int32_t* p, int32_t v, long long n, hipStream_t st);
hipError_t fill_f32(float* p, float v, long long n, hipStream_t st);
hipError_t iota_rows(int32_t* p, int rows, int n, hipStream_t st);  // p[r * n + j] = j
hipError_t add_i32(int32_t* p, int32_t v, hipStream_t st);  // *p += v (one thread)
// Decode-time loop skipping.  skip_gate, at the start of a loop k >= 2, for each of the B
// rows still in the loops (act[b] != 0): key = ||src_b - prev_b||^2 (float32 [B, d]; src
// = h_{k-1}, prev = h_{k-2}); act[b] = 0 and *live -= 1 when key < tau; prev_b = src_b
// (*live counts the rows still in the loops).  skip_restore,
// after the last loop: h_b = prev_b for the rows that left.
hipError_t skip_gate(const float* src, float* prev, int32_t* act, int32_t* live, float tau, int B, int d,
                     hipStream_t st);
hipError_t skip_restore(float* h, const float* prev, const int32_t* act, int B, int d, hipStream_t st);
hipError_t delta_keys(const float* a, const float* b, int rows, int d, float* key, hipStream_t st);
// xc[b*n + j] = (h[b*T + idx[b*n + j]] (+ add_src[same row])) + add; slot_map[b*Tmax + idx] = j
// when slot_map != nullptr.
hipError_t gather_rows(const float* h, const int32_t* idx, int B, int n, int T, int d, const u16* add,
                       float* xc, int32_t* slot_map, int Tmax, hipStream_t st, const float* add_src = nullptr);
// key[b*T + idx] = ||xc - h[idx]||^2 (when key != nullptr), then h[b*T + idx] = xc.
hipError_t scatter_rows(const float* xc, const int32_t* idx, int B, int n, int T, int d, float* h,
                        float* key, hipStream_t st);
// Top-n of each of `rows` rows of `cols` keys (ties to lower index), ascending indices.
hipError_t topk_rows(const float* keys, int rows, int cols, int n, int32_t* out, hipStream_t st);
// Quantize float32 rows [rows, hd] with a zero previous value (test entry point).
hipError_t quantize_rows(const float* x, int rows, int hd, int bits, uint8_t* codes, u16* scales,
                         hipStream_t st);

// RoPE + KV-store write.  qkv float32 [rows, (H + 2 Hkv) hd]; q_out bf16 [rows, H hd].
// Row r belongs to sequence b = r / rows_per_seq, at position pos[r] (or pos_offset +
// r % rows_per_seq when pos == nullptr).  kvw describes where K/V go:
struct KVWrite {
    int kind;             // 0: bf16 rows at (b,g,pos); 1: lazy base; 2: lazy loop-k residual
    KVLayer layer;        // destination layer (base/res pointers writable)
    int loop;             // loop k of a residual write
    const int32_t* slot_of_row;  // kind 2: slot per row (nullptr: slot = slot_base + row index in seq)
    long long slot_base;
    int32_t* slot_map_k;  // kind 2 decode: slot map of loop k to write (nullptr: already written)
    int keep_codes;       // leave int8/int4 codes and their scales in the store untouched
    const int32_t* dpos;  // decode: device position t (replaces pos_offset; slot = slot_base + t + row)
    // kinds 1 and 2, decode: also write the row's float16 reconstruction (the base's at
    // loop 1, loop k's for kind 2) into this window ring (plain rows, position p at row
    // p % ring.Tmax), when ring_on != 0.
    KVLayer ring;
    int ring_on;
    // decode (kinds 1 and 2): float32 [B][2][Hkv][hd] reconstruction of the row at the
    // previous loop of this layer (read by kind 2) and at this loop (written), in place
    // of re-reading base + residuals through the slot maps.
    float* tok_recon;
    // decode (every row at position *dpos): cos and sin of the rotation angles of that
    // position, [hd/2][2] (rope_angles), in place of evaluating them per element
    const float* rope_cs;
    // prefill: cos and sin of every prompt position p < rope_rows, [p][hd/2][2]
    // (rope_table, the same float64 evaluation rounded once), in place of evaluating
    // them per element.  nullptr: evaluated per element.
    const float* rope_tab;
    int rope_rows;
    // kind 2 decode with loop skipping: act[b] == 0 marks a sequence whose token left the
    // loops; its row stores nothing (slot map entry -1), keeps the previous loop's
    // reconstruction and puts that into the ring.  nullptr: every row stores.
    const int32_t* active;
    // set to 1 when an element this write handles (a rotated q, a rotated K or a V
    // element) is not finite or exceeds the float16 range (|x| > 65504), where the
    // float16 forms of the shared block (int8-base attention operands, decode caches,
    // float16 q) would hold inf; nullptr: no check
    uint32_t* range_flag;
};
// cos and sin (float64 evaluation, rounded to float32) of position *dpos times each
// inverse frequency into cs [hd/2][2].
hipError_t rope_angles(const int32_t* dpos, const double* inv_freq, int hd, float* cs, hipStream_t st);
// cos and sin of the rotation angles of positions 0..T-1: tab [T][hd/2][2] (float32 of
// the float64 values).
hipError_t rope_table(const double* inv_freq, int T, int hd, float* tab, hipStream_t st);
// q_half: q_out receives float16 bits instead of bfloat16 (decode, for the float16 MFMA
// attention kernels, which then take q with one rounding).
hipError_t rope_kv_write(const float* qkv, int rows, int rows_per_seq, const int32_t* pos,
                         int pos_offset, int H, int Hkv, int hd, const double* inv_freq, u16* q_out,
                         const KVWrite& kvw, hipStream_t st, int q_half = 0);

// Element e of one token's K (kv = 0, rotated by the angle of pair e % (hd/2), cosine c,
// sine sn) or V (kv = 1) row of KV head g into the store as w describes.  src: the
// token's float32 projections [(H + 2 Hkv) hd]; b: its sequence, pos: its position,
// iseq: its row within the sequence's rows of this call.  Threads e = 0..hd-1 of a
// (token, kv, g) must be consecutive lanes of one wave from a 32-lane boundary: groups
// of 32 quantize together.  `lead` (one thread per call) writes the slot map entry.
// Returns the element's reconstruction at this write's loop (the value the store and
// the window ring now hold before their 16-bit rounding; 0 for an int8 base row whose
// codes are kept, outside decode).
__device__ __forceinline__ float kv_write_elem(const float* __restrict__ src, int H, int Hkv, int hd, int b, int g,
                                              int kv, int e, int pos, int iseq, float c, float sn, const KVWrite& w,
                                              bool lead) {
    const int half = hd / 2;
    float x;
    if (kv == 0) {
        const int i = e % half;
        const float x1 = src[(H + g) * hd + i], x2 = src[(H + g) * hd + i + half];
        x = e < half ? rope_lo(x1, x2, c, sn) : rope_hi(x1, x2, c, sn);
    } else {
        x = src[(H + Hkv + g) * hd + e];
    }
    if (w.range_flag && !(fabsf(x) <= 65504.f)) *w.range_flag = 1u;
    const KVLayer& L = w.layer;
    const long long slot = w.slot_base + (w.dpos ? *w.dpos : 0) + iseq;
    const long long row = kv_row(L, b, g, pos);
    const long long idx = kv == 0 ? row * hd + e : v_elem(L, b, g, pos, e);
    // decode: this row's reconstruction at the current loop, carried to the next loop
    float* tr = w.tok_recon ? w.tok_recon + (((long long)b * 2 + kv) * Hkv + g) * hd + e : nullptr;
    auto ring_write = [&](float recon) {
        const KVLayer& Rg = w.ring;
        const int rp = pos % Rg.Tmax;
        const long long ri = kv == 0 ? kv_row(Rg, b, g, rp) * hd + e : v_elem(Rg, b, g, rp, e);
        ((u16*)Rg.base[kv])[ri] = f2h_bits(recon);
    };
    if (w.kind == 0 || (w.kind == 1 && L.base_bits == 16)) {
        const u16 xb = f2bf(x);
        ((u16*)L.base[kv])[idx] = xb;
        if (tr) *tr = bf2f(xb);
        if (w.kind == 1 && w.ring_on) ring_write(bf2f(xb));
        return bf2f(xb);
    } else if (w.kind == 1) {  // int8 base: residual against a zero reconstruction
        float recon;
        if (!w.keep_codes) {
            u16 sb;
            const int q = quant_group32(x, 127, &sb);
            ((int8_t*)L.base[kv])[idx] = (int8_t)q;
            if ((e & 31) == 0) {
                const long long si = kv == 0 ? row * (hd / 32) + e / 32 : v_scale_idx(L, b, g, pos, e / 32);
                ((u16*)L.base_scale[kv])[si] = sb;
            }
            recon = (float)q * h2f(sb);
        } else {
            recon = (tr || w.ring_on) ? kv_base_elem(L, kv, b, g, pos, e) : 0.f;
        }
        if (tr) *tr = recon;
        if (w.ring_on) ring_write(recon);
        return recon;
    } else if (w.active && !w.active[b]) {  // the token left the loops: carried row
        const float recon = tr ? *tr : kv_recon_elem(L, kv, b, g, pos, e, w.loop - 1);
        if (w.ring_on) ring_write(recon);
        if (w.slot_map_k && lead) w.slot_map_k[(long long)b * L.Tmax + pos] = -1;
        return recon;
    } else {
        const long long rr = res_row(L, b, g, slot);
        float recon;  // the row's loop-k reconstruction
        if (L.res_bits == 16) {
            const u16 xb = f2bf(x);
            ((u16*)L.res[w.loop - 2][kv])[rr * hd + e] = xb;
            recon = bf2f(xb);
        } else {
            const float prev = tr ? *tr : kv_recon_elem(L, kv, b, g, pos, e, w.loop - 1);
            if (!w.keep_codes) {
                u16 sb;
                const int qmax = (1 << (L.res_bits - 1)) - 1;
                const int q = quant_group32(x - prev, qmax, &sb);
                if ((e & 31) == 0) ((u16*)L.res_scale[w.loop - 2][kv])[rr * (hd / 32) + e / 32] = sb;
                if (L.res_bits == 8) {
                    ((int8_t*)L.res[w.loop - 2][kv])[rr * hd + e] = (int8_t)q;
                } else {
                    const int other = __shfl_xor(q, 1);
                    if ((e & 1) == 0)
                        ((uint8_t*)L.res[w.loop - 2][kv])[rr * (hd / 2) + e / 2] = (uint8_t)((q & 0xF) | ((other & 0xF) << 4));
                }
                recon = prev + (float)q * h2f(sb);
            } else {  // codes already in the store
                recon = kv_apply_res(L, kv, b, g, w.loop, (int)slot, e, prev);
            }
        }
        if (tr) *tr = recon;
        if (w.ring_on) ring_write(recon);
        if (w.slot_map_k && lead) w.slot_map_k[(long long)b * L.Tmax + pos] = (int32_t)slot;
        return recon;
    }
}

// ---- GEMM (k_gemm.hip).  C = A[M,K] * W[N,K]^T, bf16 inputs, fp32 accumulation.
enum Epi { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2, EPI_GELU = 3 };
// STORE/ADD: c float32 [M, N] (ldc = N).  SWIGLU: W = [gate (N rows); up (N rows)],
// out bf16 [M, N].  GELU: out bf16 [M, N].
hipError_t gemm(const u16* A, const u16* W, int M, int N, int K, int epi, float* c, u16* out_bf,
                hipStream_t st);
// M <= 16 only: C = (RMSNorm(X) * gain)[M,K] * W[N,K]^T with X float32 rows; the norm
// is folded into the GEMM (A operand bf16(X * gain), rows scaled by 1/rms at the end).
hipError_t gemm_rmsnorm(const float* X, const u16* gain, float eps, const u16* W, int M, int N, int K, int epi,
                        float* c, u16* out_bf, hipStream_t st);

// Decode-sized products (M <= 8 rows, K % 64 == 0, N % 8 == 0) with the RMSNorm
// carried between kernels: a producer adds its product into the residual stream x
// and leaves xg = x * next_gain plus per-workgroup row sums of x^2 (ps, [nparts][8]);
// the consumer multiplies xg by W and scales by 1 / sqrt(sum(ps) / K + eps).
// Weights (Wp) and activations (xg, A, and the activation outputs) are in the
// lane-packed order of pk_index (weights: rows = N, or 2N for SwiGLU's [gate; up]).
// Operands are float16: the weights as converted from bf16 by pack_weights (exact for
// magnitudes in [2^-17, 65504]) and every activation rounded once from float32.
struct FoldIO {
    const float* ps_in;    // NORM: partial sums of x^2 [nparts][8]
    int nparts;
    float eps;
    const u16* add_vec;    // PREP: bf16 [N] added to x after the product (nullptr: none)
    const float* add_rows; // PREP: float32 [M, N] added to x after the product, before add_vec
    float* x_save;         // PREP: float32 [M, N] receives x after the product, before the adds
    const u16* next_gain;  // PREP: bf16 [N] gain of the next RMSNorm
    u16* xg_out;           // PREP: float16 [M, N], lane-packed
    float* ps_out;         // PREP: [N / 8][8]
    const int32_t* live;   // nonzero *live or nullptr: run; *live == 0: return at once
};
bool gemm_fold_supported(int M, int N, int K);
hipError_t gemm_fold_norm(const u16* xg, const float* ps, int nparts, float eps, const u16* Wp, int M, int N, int K,
                          int epi, float* c, u16* out_bf, hipStream_t st, const int32_t* live = nullptr);
// x[M, N] += A W^T (then + add_rows, then + add_vec); with next_gain also writes xg_out and
// ps_out (N / 8 parts); x_save (with next_gain) receives x before add_rows and add_vec.
hipError_t gemm_fold_add(const u16* A, const u16* Wp, int M, int N, int K, float* x, const u16* add_vec,
                         const u16* next_gain, u16* xg_out, float* ps_out, hipStream_t st,
                         const float* add_rows = nullptr, float* x_save = nullptr, const int32_t* live = nullptr);
// Row-major bf16 W [rows, K] -> lane-packed float16 Wp (rows % 8 == 0, K % 64 == 0).
hipError_t pack_weights(const u16* W, long long rows, int K, u16* Wp, hipStream_t st);
// x += add (optional); xg = x * gain as lane-packed float16; ps[0][r] = sum of x^2 of
// row r.
hipError_t norm_prep(float* x, const u16* add, const u16* gain, int rows, int d, u16* xg, float* ps,
                     hipStream_t st);

// ---- attention (k_attn.hip)
// Dense causal prefill over a bf16 (or int8-base) layer: q bf16 [B*T, H*hd] (row b*T+i),
// out bf16 [B*T, H*hd], lse float32 [B, H, T] (log2 units of the scaled scores).
hipError_t attn_prefill(const u16* q, const KVLayer& kv, int B, int T, int H, u16* out, float* lse,
                        hipStream_t st);
// Column mass of loop-1 attention: mass float32 [B, Hkv, T].
hipError_t column_mass(const u16* q, const KVLayer& kv, const float* lse, int B, int T, int H,
                       float* mass, hipStream_t st);

// Row attention over explicit column sets (decode and token-sparse prefill).
struct RowsAttn {
    const u16* q;          // bf16 [B * n_rows, H * hd] (float16 when q_half != 0)
    int q_half;            // q holds float16 bits (decode: the float16 MFMA kernels take it as is)
    const int32_t* qpos;   // [B * n_rows] positions (nullptr: all rows at `pos`)
    int pos;
    int B, n_rows, H;
    KVLayer kv;
    int k_loop;            // reconstruction loop (1 = base / plain rows)
    const int32_t* cols;   // sparse: [B][Hkv][n_cols] ascending (nullptr: dense causal)
    int n_cols, window;
    int chunk, n_splits;   // columns per split, splits per row
    float* part;           // [B*n_rows][Hkv][n_splits][G][hd + 2]
    u16* out;              // bf16 [B * n_rows, H * hd]
    const int32_t* lens;   // dense: columns per (b, g) (nullptr: pos + 1 for all)
    const int32_t* dpos;   // decode: device position t (replaces pos)
    // Two-segment sparse decode (seg_split > 0): splits [0, seg_split) run over kv, the
    // float16 reconstruction of the column set S (row i = column cols[i]; rows with
    // cols[i] > pos - window are masked); splits from seg_split on run over kv2, a
    // ring of float16 window rows (position p at row p % kv2.Tmax), keys taken from
    // position (max(0, pos-window+1) & ~7) with those below the window masked.
    KVLayer kv2;
    int seg_split;
    // Decode (one row per sequence at position *dpos) with fuse_kv: q comes from the
    // float32 projections qkv [B][(H + 2 Hkv) hd], rotated here with rope_cs
    // ([hd/2][cos, sin] of the position), and that token's K/V row is written as kvw
    // describes (the work a separate rope_kv_write launch does otherwise): by the
    // new-key split below when it is on, else first by the workgroup whose keys include
    // the new position.
    const float* qkv;
    const float* rope_cs;
    KVWrite kvw;
    int fuse_kv;
    // New-key split of the two-segment decode (fuse_kv; nk_split = n_splits - 1, 0: off):
    // split nk_split of every (b, g) writes the new token's K/V row and forms that one
    // key's partial from the values it wrote (score in float32 from the float16 q and K,
    // weight 1, output the float16 V); the window splits stop below the new key.
    int nk_split;
    // Difference-corrected sparse attention: the normalized output o of query row
    // (b, i), heads h, meets a correction row (DIFF_NONE: out = o).
    //   DIFF_ADD32  out = o + d32[b * n_rows + i]
    //   DIFF_SET32  d32[b * n_rows + i] = o, and out = o
    //   DIFF_SUB32  d32[b * n_rows + i] -= o; out is not written
    //   DIFF_ADD16  out = o + d16[b][qpos]
    //   DIFF_OUT16  d16[b][qpos] = out - o; out is read, not written
    // d32 is float32 [B * n_rows][H * hd]; d16 float16 [B][d_rows][H * hd].  The
    // combine takes every mode; attn_rows_prefill takes ADD16 and OUT16.
    int diff_mode;
    float* d32;
    u16* d16;
    int d_rows;
    // Decode-time loop skipping: *live == 0 (no sequence left in the loops) makes the
    // two-segment sparse launch do only its new-token K/V write and the merge return at
    // once.  nullptr: always run.
    const int32_t* live;
};
enum { DIFF_NONE = 0, DIFF_ADD32, DIFF_SET32, DIFF_SUB32, DIFF_ADD16, DIFF_OUT16 };
// Write loop-k reconstructions as float16 rows into kc [B*Hkv][ncap][hd] and
// 8-key-interleaved vc [B*Hkv][ncap/8][hd][8] (rows past the count are zero):
//  GATHER_ALL_S:  row i = column cols[i] of the (b, g) column set, i < n_cols;
//  GATHER_RING:   positions p in [roundup8(max(0, T - ncap)), T) for T = pos + 1,
//                 each at row p % ncap (the window ring at the end of prefill; other
//                 rows are left as they are).
enum { GATHER_ALL_S = 1, GATHER_RING = 3 };
hipError_t gather_recon(const RowsAttn& a, int mode, int ncap, u16* kc, u16* vc, hipStream_t st);
// Token-sparse prefill rows (rows_per_seq > 1, hd 128): every kept row q of sequence b
// (position qpos) attends over the cache rows of sc whose column cols[r] <= qpos - window
// and over the positions (qpos - window, qpos] of fr (float16 plain layers: K rows, V
// 8-key interleaved); writes `out` directly.  hipErrorInvalidValue if the shape is not
// taken.
hipError_t attn_rows_prefill(const RowsAttn& a, const KVLayer& sc, const KVLayer& fr, hipStream_t st);
// attn_rows_main writes the per-split partials; attn_rows_combine merges them into `out`.
hipError_t attn_rows_main(const RowsAttn& a, hipStream_t st);
// packed_out: out in the lane-packed order of the decode products (at most 8 rows), as
// float16.
hipError_t attn_rows_combine(const RowsAttn& a, hipStream_t st, bool packed_out = false);

}  // namespace lk
