// Split-K grouped-query decode attention (gfx950, wave64, bf16 MFMA 16x16x16).
//
// One work item = (sequence b, KV head j, split s of the key axis).  The item's
// workgroup serves all G = Hq/Hkv query heads of KV head j from one read of the
// K/V tiles (Unsloth article 二.2: query heads address their KV head by index,
// never by a broadcast copy).  Keys are processed in 16-key subtiles, one
// subtile per wave at a time, with an online softmax (Roofline reply 四:
// FlashAttention-style tiling; the score row never reaches HBM).  Each item
// leaves a partial (running max m, running sum l, unnormalised output O); a
// second kernel merges the splits of each query head in split order, so the
// result is bit-reproducible.  Workgroups never wait on or signal each other:
// a device-scope fence per workgroup (what a last-arriver merge needs for the
// partials to be visible across XCDs) writes back the XCD's L2 and serialises,
// which costs far more than the kernel boundary does.
//
// MFMA mapping (16x16x16 bf16, fp32 accumulate):
//   scores^T[key][head] = K_tile[key][dims] x q^T[dims][head]  (M = 16 keys,
//       N = 16 heads (G used), K = 16 dims per instruction).  Lane (r, g)
//       (r = lane % 16, g = lane / 16) feeds key r, dims 32g + 4kb + i of its
//       own 64 contiguous bytes of the K row, and receives the scores of head r
//       for keys 4g..4g+3 -- which is exactly the A-operand layout of
//   O[head][dim] += P[head][key] x V[key][dim]  (M = heads, N = 16 dims, K = 16
//       keys).  V is cached transposed ([dim][position]) so that lane (r, g)
//       reads keys 4g..4g+3 of dimension 16nt + r as one 8-byte load.
// q and P are split into bf16 hi + lo parts (two MFMAs each), which carries
// them at about 16 significant bits; K and V are exact bf16, products are exact
// in fp32.  Scores are in log2 units (q is pre-scaled by log2(e)/sqrt(hd)).
#pragma once
#include "common.h"

struct AttnArgs {
    const float* q;          // [B][Hq][hd] fp32
    const uint16_t* kc;      // [B][Hkv][cap][hd]
    const uint16_t* vc;      // [B][Hkv][hd][cap]
    const int* pos;          // [B]
    int cap, hq, hkv, batch, max_pos;
    int nsplit;              // splits per (b, j)
    int T;                   // keys per split (multiple of 4)
    int nsplit_max;          // partial-buffer stride
    float qscale;            // log2(e) / sqrt(hd)
    float* pm; float* pl;    // [B][Hq][nsplit_max]
    float* po;               // [B][Hq][nsplit_max][hd]
    float* o;                // [B][Hq][hd] fp32 (merge kernel output)
};

I4D_DEVINL u32x4 nt_load_k(const u32x4* p) { return ld_g_nt(p); }
I4D_DEVINL u32x2 nt_load_v(const u32x2* p) { return ld_g_nt(p); }

I4D_DEVINL s4 pack_bf16x4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
    s4 r; r[0] = (short)a; r[1] = (short)b; r[2] = (short)c; r[3] = (short)d; return r;
}
I4D_DEVINL s4 dwords_to_s4(u32 lo, u32 hi) { return __builtin_bit_cast(s4, u32x2{lo, hi}); }

// Number of keys attended by sequence b (pos + 1), or 0 if pos is invalid.
I4D_DEVINL int keys_of(const AttnArgs& a, int b) {
    const int p = a.pos[b];
    return (p >= 0 && p <= a.max_pos && p < a.cap) ? p + 1 : 0;
}

// LDS bytes used by attn_item with NT threads.
template <int HD, int NT>
__host__ __device__ constexpr int attn_lds_bytes() { return (NT / 64) * (16 * HD + 32) * 4 + (HD / 16) * 2 * 64 * 8; }

template <int HD, int NT>
I4D_DEVINL void attn_item(const AttnArgs& a, int item, char* lds) {
    constexpr int NW = NT / 64, NKB = HD / 16, DPL = HD / 4;   // DPL: dims per lane group
    const int tid = i4d_tid(), lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int G = a.hq / a.hkv;
    const int s = item % a.nsplit;
    const int j = (item / a.nsplit) % a.hkv;
    const int b = item / (a.nsplit * a.hkv);
    const int nk = keys_of(a, b);
    const int t_s = s * a.T;
    const int t_e = min(t_s + a.T, nk);
    const int nsub = (t_e > t_s) ? (t_e - t_s + 15) / 16 : 0;

    // q^T operand (hi, lo) for head r of this group, dims DPL*g + 4kb + i, kept
    // in LDS (every wave of the workgroup uses the same operands): [kb][lane]
    // s4 pairs after the per-wave areas.  Vector loads from a clamped head,
    // zeroed for padding heads r >= G.
    s4* qop = (s4*)(lds + NW * (16 * HD + 32) * 4);
    if (wave == 0) {
        const f4* qp = (const f4*)(a.q + ((size_t)(b * a.hq + j * G + min(r, G - 1)) * HD) + DPL * g);
        f4 qv[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qv[kb] = qp[kb];    // this layer's q, first read after it was written
        const float qs = (r < G) ? a.qscale : 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            uint16_t hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = qv[kb][i] * qs;
                hv[i] = f32_to_bf16(v);
                lv[i] = f32_to_bf16(v - bf16_to_f32(hv[i]));
            }
            qop[(2 * kb) * 64 + lane] = pack_bf16x4(hv[0], hv[1], hv[2], hv[3]);
            qop[(2 * kb + 1) * 64 + lane] = pack_bf16x4(lv[0], lv[1], lv[2], lv[3]);
        }
    }
    __syncthreads();

    const uint16_t* kbase = a.kc + (size_t)(b * a.hkv + j) * a.cap * HD;
    const uint16_t* vbase = a.vc + (size_t)(b * a.hkv + j) * HD * a.cap;

    float m = -INFINITY, lsum = 0.f;
    f4 O[NKB];
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt) O[nt] = f4{0.f, 0.f, 0.f, 0.f};

    // One 16-key subtile: K rows (key t0 + r, dims DPL*g ..) and V^T runs
    // (dim 16nt + r, keys t0 + 4g .. t0 + 4g + 3).  Addresses are clamped into
    // the cache so every load is issued unconditionally; keys outside
    // [t_s, t_e) are zeroed when the subtile is consumed.
    auto load_sub = [&](int st, u32x4 (&kr)[NKB / 2], u32x2 (&vr)[NKB]) {
        const int t0 = t_s + 16 * st;
        const int tk = min(t0 + r, a.cap - 1);
        const u32x4* kp = (const u32x4*)(kbase + (size_t)tk * HD + DPL * g);
#pragma unroll
        for (int mm = 0; mm < NKB / 2; ++mm) kr[mm] = nt_load_k(kp + mm);
        const int tv = min(t0 + 4 * g, a.cap - 4);
#pragma unroll
        for (int nt = 0; nt < NKB; ++nt) vr[nt] = nt_load_v((const u32x2*)(vbase + (size_t)(16 * nt + r) * a.cap + tv));
    };

    auto compute_sub = [&](int st, const u32x4 (&kr)[NKB / 2], const u32x2 (&vr)[NKB]) {
        const int t0 = t_s + 16 * st;
        const int tv = t0 + 4 * g;
        const bool kvalid = t0 + r < t_e;               // this lane's K row
        const int vvalid = t_e - tv;                    // keys of this lane's V run in range
        // scores^T for keys 4g..4g+3 of head r
        f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 w = kr[kb >> 1];
            if (!kvalid) w = u32x4{0, 0, 0, 0};
            const s4 kop = (kb & 1) ? dwords_to_s4(w.z, w.w) : dwords_to_s4(w.x, w.y);
            sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kop, qop[(2 * kb) * 64 + lane], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kop, qop[(2 * kb + 1) * 64 + lane], sc, 0, 0, 0);
        }
        float sv[4] = {sc[0], sc[1], sc[2], sc[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tv + i >= t_e) sv[i] = -INFINITY;
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mnew = fmaxf(m, mx);                // finite: the subtile has a valid key
        const float alpha = exp2f(m - mnew);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = exp2f(sv[i] - mnew);
        lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m = mnew;
        // rescale O rows (heads 4g + i) by their alpha
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = shfl_f(alpha, 4 * g + i);
#pragma unroll
            for (int nt = 0; nt < NKB; ++nt) O[nt][i] *= ai;
        }
        uint16_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ph[i] = f32_to_bf16(p[i]);
            pl[i] = f32_to_bf16(p[i] - bf16_to_f32(ph[i]));
        }
        const s4 pho = pack_bf16x4(ph[0], ph[1], ph[2], ph[3]);
        const s4 plo = pack_bf16x4(pl[0], pl[1], pl[2], pl[3]);
        const u32 vm0 = vvalid >= 2 ? 0xFFFFFFFFu : (vvalid == 1 ? 0x0000FFFFu : 0u);
        const u32 vm1 = vvalid >= 4 ? 0xFFFFFFFFu : (vvalid == 3 ? 0x0000FFFFu : 0u);
#pragma unroll
        for (int nt = 0; nt < NKB; ++nt) {
            const s4 vop = dwords_to_s4(vr[nt].x & vm0, vr[nt].y & vm1);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pho, vop, O[nt], 0, 0, 0);
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vop, O[nt], 0, 0, 0);
        }
    };

    // Two subtiles in flight per wave.  Each "prefetch; compute" block issues
    // its loads unconditionally, so the wait before a compute only covers the
    // buffer it reads; the last subtile of the wave is computed on its own.
    u32x4 kr0[NKB / 2], kr1[NKB / 2];
    u32x2 vr0[NKB], vr1[NKB];
    int st = wave;
    if (st < nsub) {
        load_sub(st, kr0, vr0);
        for (;;) {
            if (st + NW >= nsub) { compute_sub(st, kr0, vr0); break; }
            load_sub(st + NW, kr1, vr1);
            compute_sub(st, kr0, vr0);
            st += NW;
            if (st + NW >= nsub) { compute_sub(st, kr1, vr1); break; }
            load_sub(st + NW, kr0, vr0);
            compute_sub(st, kr1, vr1);
            st += NW;
        }
    }

    // per-wave state -> LDS: wm[16], wl[16], wo[16][HD] per wave
    float* wbase = (float*)lds + wave * (16 * HD + 32);
    float lt = lsum;
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    if (g == 0) { wbase[r] = m; wbase[16 + r] = lt; }
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) wbase[32 + (4 * g + i) * HD + 16 * nt + r] = O[nt][i];
    __syncthreads();

    // combine the waves; write this split's partial
    const size_t hrow0 = (size_t)(b * a.hq + j * G);
    for (int idx = tid; idx < G * HD; idx += NT) {
        const int h = idx / HD, d = idx - h * HD;
        const float* lw = (const float*)lds;
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, lw[w * (16 * HD + 32) + h]);
        float acc = 0.f, L = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < NW; ++w) {
                const float* wb = lw + w * (16 * HD + 32);
                const float e = exp2f(wb[h] - M);
                acc = fmaf(wb[32 + h * HD + d], e, acc);
                L = fmaf(wb[16 + h], e, L);
            }
        }
        const size_t pidx = (hrow0 + h) * a.nsplit_max + s;
        st_dev(a.po + pidx * HD + d, acc);
        if (d == 0) { st_dev(a.pm + pidx, M); st_dev(a.pl + pidx, L); }
    }
    __syncthreads();       // the wave area of LDS is reused by the next item
}

// Merge the splits of query heads: o = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^(m_s - max m), in split order.  Each group of HD threads of the
// workgroup merges head bh0 + group (if < nheads); every thread of the
// workgroup must call this (it synchronises).  LDS: (NT/HD) * 2 * nsplit floats.
template <int HD, int NT>
I4D_DEVINL void attn_merge_heads(const AttnArgs& a, int bh0, int nheads, float* lds) {
    const int g = i4d_tid() / HD, lt = i4d_tid() - g * HD;
    const int bh = bh0 + g;
    const bool valid = (g < NT / HD) && (bh < nheads);
    const int ns = a.nsplit;
    const size_t prow = (size_t)bh * a.nsplit_max;
    float* sm = lds + g * 2 * ns;      // split maxima, then weights
    float* sl = sm + ns;               // split sums
    if (valid)
        for (int ss = lt; ss < ns; ss += HD) { sm[ss] = ld_dev(a.pm + prow + ss); sl[ss] = ld_dev(a.pl + prow + ss); }
    __syncthreads();
    float M = -INFINITY, L = 0.f;
    if (valid) {
        for (int ss = 0; ss < ns; ++ss) M = fmaxf(M, sm[ss]);
        if (M != -INFINITY)
            for (int ss = 0; ss < ns; ++ss) L = fmaf(sl[ss], exp2f(sm[ss] - M), L);
    }
    const float inv = (L > 0.f) ? 1.0f / L : 0.f;
    __syncthreads();
    if (valid)
        for (int ss = lt; ss < ns; ss += HD) sm[ss] = (M != -INFINITY) ? exp2f(sm[ss] - M) * inv : 0.f;
    __syncthreads();
    if (valid) {
        const float* src = a.po + prow * HD + lt;
        float acc = 0.f;
#pragma unroll 16
        for (int ss = 0; ss < ns; ++ss) acc = fmaf(sm[ss], ld_dev(src + (size_t)ss * HD), acc);
        st_dev(a.o + (size_t)bh * HD + lt, acc);
    }
    __syncthreads();
}
