// Split-K grouped-query decode attention (gfx950, wave64, bf16 MFMA 16x16x16).
//
// One work item = (sequence b, KV head j, split s of the key axis).  The item's
// workgroup serves all G = Hq/Hkv query heads of KV head j from one read of the
// K/V tiles (Unsloth article 二.2: query heads address their KV head by index,
// never by a broadcast copy).  Keys are processed in 16-key subtiles with an
// online softmax (Roofline reply 四: FlashAttention-style tiling; the score row
// never reaches HBM).  Subtile st of an item belongs to wave st % NW.
//
// Loads.  A wave issues the K/V loads of all its subtiles of a round (up to
// NSW of them) before computing any, so an item costs about one memory round
// trip; the streaming kernel (stream.hip) issues round 0 before it waits for
// this step's q, k and v, because the cached history does not depend on the
// q/k/v phase.  The one key that does -- the new token's, at position pos[b] --
// is read from the exchange vector that the q/k/v epilogue writes, and patched
// into the registers once it has arrived; cache lines loaded earlier may hold
// the old contents of that slot.
//
// Merge.  Each item leaves a partial (running max m, running sum l,
// unnormalised O); the last of the nsplit workgroups of (b, j) to finish
// (an arrival counter) merges the splits in split order, so the result is
// bit-reproducible.  Partials are written through to memory and the counter is
// incremented only after those stores completed, so the merging workgroup sees
// every split; no cache-writeback fence is needed.
//
// MFMA mapping (16x16x16 bf16, fp32 accumulate):
//   scores^T[key][head] = K_tile[key][dims] x q^T[dims][head]  (M = 16 keys,
//       N = 16 heads (G used), K = 16 dims per instruction).  Lane (r, g)
//       (r = lane % 16, g = lane / 16) feeds key r, dims 32(kb/2) + 8g +
//       4(kb%2) + i (for each 16-byte load the four lanes of key r read 64
//       contiguous bytes of its row; q^T uses the same dim order), and
//       receives the scores of head r for keys 4g..4g+3 -- which is exactly the
//       A-operand layout of
//   O[head][dim] += P[head][key] x V[key][dim]  (M = heads, N = 16 dims, K = 16
//       keys).  V is cached dim-major inside each 16-position tile so that
//       lane (r, g) reads keys 4g..4g+3 of dimension 16nt + r as one 8-byte
//       load.
// q and P are split into bf16 hi + lo parts (two MFMAs each), which carries
// them at about 16 significant bits; K and V are exact bf16, products are exact
// in fp32.  Scores are in log2 units (q is pre-scaled by log2(e)/sqrt(hd)).
#pragma once
#include "common.h"

// Where the 16-position tiles of a KV cache live.  pages == nullptr: the
// contiguous layout [row][Hkv][cap/16] (the caller's cap and Hkv).  Otherwise a
// pool of pages of `page_tiles` tiles, laid out [page][Hkv][page_tiles], and a
// table [row][pps] of page ids; an id outside 0..n_pages-1 reads page 0 and
// raises I4D_DEV_BAD_PAGE in *status.
struct KvMap {
    const int* pages;
    int page_tiles, n_pages, pps;
};

// Element offset of tile t of (cache row r, KV head j), for tiles of 16 * hd
// elements.  bad: set when the page id was out of range (page 0 was used).
I4D_DEVINL size_t kv_tile_off(const KvMap& m, int cap, int hkv, int hd, int r, int j, int t, bool& bad) {
    if (m.pages == nullptr) return ((size_t)(r * hkv + j) * cap + (size_t)t * 16) * hd;
    int pg = ld_g(m.pages + (size_t)r * m.pps + t / m.page_tiles);
    bad = pg < 0 || pg >= m.n_pages;
    if (bad) pg = 0;
    return ((size_t)(pg * hkv + j) * m.page_tiles + t % m.page_tiles) * 16 * hd;
}

struct AttnArgs {
    const float* q;          // [B][Hq][hd] fp32
    const uint16_t* kc;      // [B][Hkv][cap/16][hd/32][16][32]
    const uint16_t* vc;      // [B][Hkv][cap/16][hd][16]
    const uint16_t* kvn;     // [B][Hkv][2][hd]: the new token's bf16 k (row 0) and v (row 1)
    const int* pos;          // [B]
    int cap, hq, hkv, batch, max_pos;
    int kvb;                 // 1: sequence b has cache b; 0: every entry shares cache 0 (a prompt chunk)
    int nsplit;              // splits per (b, j)
    int T;                   // keys per split (multiple of 16)
    int pstride;             // partial-buffer stride per head (multiple of 32 splits)
    float qscale;            // log2(e) / sqrt(hd)
    float* pm; float* pl;    // [B][Hq][pstride]
    float* po;               // [B][Hq][pstride][hd]
    int* cnt;                // [B][Hkv] arrival counters, zero between calls
    float* o;                // [B][Hq][hd] fp32 merged output
    KvMap pg;                // paged caches (pg.pages == nullptr: contiguous)
    int* status;             // workspace status word (I4D_DEV_BAD_PAGE)
};

I4D_DEVINL u32x4 nt_load_k(const u32x4* p) { return ld_g_nt(p); }
I4D_DEVINL u32x2 nt_load_v(const u32x2* p) { return ld_g_nt(p); }

I4D_DEVINL s4 pack_bf16x4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
    s4 r; r[0] = (short)a; r[1] = (short)b; r[2] = (short)c; r[3] = (short)d; return r;
}
I4D_DEVINL s4 dwords_to_s4(u32 lo, u32 hi) { return __builtin_bit_cast(s4, u32x2{lo, hi}); }

// Number of keys attended by sequence b (pos + 1), or 0 if pos is invalid.
I4D_DEVINL int keys_of(const AttnArgs& a, int b) {
    const int p = ld_g(a.pos + b);
    return (p >= 0 && p <= a.max_pos && p < a.cap) ? p + 1 : 0;
}

// LDS bytes used by the attention of one workgroup of NT threads: per-wave
// partial states, then the q operand (the merge reuses the per-wave area).
template <int HD, int NT>
__host__ __device__ constexpr int attn_lds_bytes() { return (NT / 64) * (16 * HD + 32) * 4 + (HD / 16) * 2 * 64 * 8; }

// Subtiles a wave holds in registers per round.
template <int NT> struct AttnNsw { static constexpr int v = NT >= 512 ? 3 : 5; };

struct AttnGeo {
    int b, j, s, t_s, t_e, nsub, kpos;     // kpos: the new key's position, -1 if none
};

// nk: keys of the item's sequence (keys_of), when the caller already knows it
I4D_DEVINL AttnGeo attn_geo_nk(const AttnArgs& a, int item, int nk) {
    AttnGeo g;
    g.s = item % a.nsplit;
    g.j = (item / a.nsplit) % a.hkv;
    g.b = item / (a.nsplit * a.hkv);
    g.t_s = g.s * a.T;
    g.t_e = min(g.t_s + a.T, nk);
    g.nsub = (g.t_e > g.t_s) ? (g.t_e - g.t_s + 15) / 16 : 0;
    g.kpos = nk - 1;
    return g;
}
I4D_DEVINL AttnGeo attn_geo(const AttnArgs& a, int item) {
    return attn_geo_nk(a, item, keys_of(a, item / (a.nsplit * a.hkv)));
}

template <int HD, int NSW>
struct AttnRegs {
    u32x4 k[NSW][HD / 32];
    u32x2 v[NSW][HD / 16];
};

// K (key t0 + r, dims 32mm + 8g .. + 8) and V (dim 16nt + r, keys t0 + 4g ..
// t0 + 4g + 3) of subtile st, from the cache's 16-position tiles (the cache
// layout is chosen so that every load instruction reads whole cache lines).
// Subtiles start on tile boundaries (keys per split are a multiple of 16);
// keys outside the item are masked when the subtile is used.
// A slot past the item (live = false) reads one 16-byte word of the cache for
// every lane instead: the loads stay unconditional, so the compiler can count
// them exactly, but cost one cache line each.
// PAGED: the cache is a page pool (a.pg), compiled separately so that the
// contiguous kernel keeps its plain address arithmetic.
template <int HD, bool PAGED>
I4D_DEVINL void attn_load_sub(const AttnArgs& a, const AttnGeo& g, int st, bool live, size_t poff, u32x4 (&kr)[HD / 32],
                              u32x2 (&vr)[HD / 16]) {
    constexpr int NKB = HD / 16;
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    // kbase/vbase + tile: this subtile's 16-position tile (kbase/vbase alone: a
    // slot past the item reads tile 0 of the row)
    const uint16_t* kbase;
    const uint16_t* vbase;
    size_t tile;
    if constexpr (PAGED) {
        // poff: the tile's offset in the pool, looked up ahead (attn_page_offsets)
        kbase = a.kc + poff;
        vbase = a.vc + poff;
        tile = 0;
    } else {
        kbase = a.kc + (size_t)(g.b * a.kvb * a.hkv + g.j) * a.cap * HD;
        vbase = a.vc + (size_t)(g.b * a.kvb * a.hkv + g.j) * HD * a.cap;
        tile = (size_t)((g.t_s >> 4) + st) * 16 * HD;
    }
    // K tile [HD/32][16][32]: block mm of the four lanes of key r is 64 bytes;
    // one instruction reads the 1 KB block [mm][0..15][0..31]
    const uint16_t* kp = live ? kbase + tile + r * 32 + 8 * gq : kbase;
#pragma unroll
    for (int mm = 0; mm < NKB / 2; ++mm) kr[mm] = nt_load_k((const u32x4*)(kp + (live ? 512 * mm : 0)));
    // V tile [HD][16]: one instruction reads dims 16nt..16nt+15, 512 contiguous bytes
    const uint16_t* vp = live ? vbase + tile + r * 16 + 4 * gq : vbase;
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt) vr[nt] = nt_load_v((const u32x2*)(vp + (live ? 256 * nt : 0)));
}

// Paged caches: the pool offsets of this wave's subtiles of round rnd (tile 0
// of the row for slots past the item).  Issued a round ahead, so the page-table
// reads overlap the previous round instead of preceding every K/V load.
template <int HD, int NT, int NSW>
I4D_DEVINL void attn_page_offsets(const AttnArgs& a, const AttnGeo& g, int rnd, size_t (&off)[NSW]) {
    constexpr int NW = NT / 64;
    const int wave = i4d_tid() >> 6;
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
        const int st = (rnd * NSW + i) * NW + wave;
        bool bad = false;
        off[i] = kv_tile_off(a.pg, a.cap, a.hkv, HD, g.b * a.kvb, g.j, st < g.nsub ? (g.t_s >> 4) + st : 0, bad);
        if (bad && (i4d_tid() & 63) == 0 && a.status) raise_status(a.status, I4D_DEV_BAD_PAGE);
    }
}

// Issue the loads of round r of this wave (off: the paged offsets of the round).
template <int HD, int NT, int NSW, bool PAGED = false>
I4D_DEVINL void attn_load_round(const AttnArgs& a, const AttnGeo& g, int rnd, AttnRegs<HD, NSW>& R,
                                const size_t* off = nullptr) {
    constexpr int NW = NT / 64;
    const int wave = i4d_tid() >> 6;
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
        const int st = (rnd * NSW + i) * NW + wave;
        attn_load_sub<HD, PAGED>(a, g, st, st < g.nsub, PAGED ? off[i] : 0, R.k[i], R.v[i]);
    }
}

// Replace the new key's K row and V column in subtile st's registers with the
// side-buffer values (the cached copies may predate this step's append).
template <int HD>
I4D_DEVINL void attn_patch_new(const AttnArgs& a, const AttnGeo& g, int st, u32x4 (&kr)[HD / 32], u32x2 (&vr)[HD / 16]) {
    constexpr int NKB = HD / 16, DPL = HD / 4;
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    const int t0 = g.t_s + 16 * st;
    const uint16_t* kn = a.kvn + (size_t)(g.b * a.hkv + g.j) * 2 * HD;
    if (t0 + r == g.kpos) {
#pragma unroll
        for (int mm = 0; mm < NKB / 2; ++mm) kr[mm] = ld_g((const u32x4*)(kn + 32 * mm + 8 * gq));
    }
    const int e = g.kpos - (t0 + 4 * gq);          // index of the new key in this lane's run of 4
    if (e >= 0 && e < 4) {
#pragma unroll
        for (int nt = 0; nt < NKB; ++nt) {
            const u32 nv = (u32)ld_g(kn + HD + 16 * nt + r);
            u32 lo = vr[nt].x, hi = vr[nt].y;
            if (e == 0) lo = (lo & 0xFFFF0000u) | nv;
            else if (e == 1) lo = (lo & 0x0000FFFFu) | (nv << 16);
            else if (e == 2) hi = (hi & 0xFFFF0000u) | nv;
            else hi = (hi & 0x0000FFFFu) | (nv << 16);
            vr[nt] = u32x2{lo, hi};
        }
    }
}

// One 16-key subtile st of an item: scores against the q operand (qop, the
// hi/lo bf16 parts in LDS), online-softmax update of this lane's running max m
// and sum lsum, and O += P V.  Keys at or past g.t_e are masked.
template <int HD>
I4D_DEVINL void attn_sub(const AttnGeo& g, int st, const u32x4 (&kr)[HD / 32], const u32x2 (&vr)[HD / 16], const s4* qop,
                         float& m, float& lsum, f4 (&O)[HD / 16]) {
    constexpr int NKB = HD / 16;
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    const int t_e = g.t_e;
    const int t0 = g.t_s + 16 * st;
    const int tv = t0 + 4 * gq;
    const bool kvalid = t0 + r < t_e;               // this lane's K row
    const int vvalid = t_e - tv;                    // keys of this lane's V run in range
    // scores^T for keys 4gq..4gq+3 of head r: four independent accumulators
    // (q's high and low parts, even and odd dimension blocks) so that the
    // matrix-core instructions do not wait on each other's results
    f4 sc[4] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        u32x4 w = kr[kb >> 1];
        if (!kvalid) w = u32x4{0, 0, 0, 0};
        const s4 kop = (kb & 1) ? dwords_to_s4(w.z, w.w) : dwords_to_s4(w.x, w.y);
        sc[kb & 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kop, qop[(2 * kb) * 64 + lane], sc[kb & 1], 0, 0, 0);
        sc[2 + (kb & 1)] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kop, qop[(2 * kb + 1) * 64 + lane], sc[2 + (kb & 1)], 0, 0, 0);
    }
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (sc[0][i] + sc[1][i]) + (sc[2][i] + sc[3][i]);
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
    // rescale O rows (heads 4gq + i) by their alpha
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float ai = shfl_f(alpha, 4 * gq + i);
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
}

// Two subtiles st0 and st1 (st1 may lie past the item: all its keys masked) in
// one online-softmax step, on gfx950's 16x16x32 bf16 matrix instruction.  The
// instruction pairs A and B by (lane group, element), so each operand only has
// to list the K axis in the same order on both sides:
//   scores^T[key][head]: A = the K row (lane (r, g): key r, the 8 dims of its
//     16-byte load), B = q^T (lane (r, g): head r, the same 8 dims), one
//     instruction per 32-dim block and per q part (high, low);
//   O[head][dim] += P V: element j of lane group g is key 4g + j of subtile
//     st0 for j < 4, key 4g + j - 4 of st1 otherwise: A = P (lane (r, g): head
//     r), B = V (lane (r, g): dim 16 nt + r), so both subtiles take two
//     instructions per 16-dim tile (P high, P low).
// q32: the q operand in LDS, q32[(2 mm + p) * 64 + lane] = part p (0 high, 1
// low bf16) of dims 32 mm + 8 g .. + 7 of head r.  Same arithmetic per key as
// attn_sub, up to summation order.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

I4D_DEVINL bf16x8 as_bf16x8(u32 a, u32 b, u32 c, u32 d) { return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d}); }

template <int HD>
I4D_DEVINL void attn_sub2(const AttnGeo& g, int st0, int st1, const u32x4 (&kr0)[HD / 32], const u32x2 (&vr0)[HD / 16],
                          const u32x4 (&kr1)[HD / 32], const u32x2 (&vr1)[HD / 16], const u32x4* q32,
                          float& m, float& lsum, f4 (&O)[HD / 16]) {
    constexpr int NKB = HD / 16, NMM = HD / 32;
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    const int t_e = g.t_e;
    const int t00 = g.t_s + 16 * st0, t01 = g.t_s + 16 * st1;
    const int tv0 = t00 + 4 * gq, tv1 = t01 + 4 * gq;
    const bool kv0 = t00 + r < t_e, kv1 = t01 + r < t_e;
    f4 s0[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    f4 s1[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm) {
        const bf16x8 qh = __builtin_bit_cast(bf16x8, q32[(2 * mm) * 64 + lane]);
        const bf16x8 ql = __builtin_bit_cast(bf16x8, q32[(2 * mm + 1) * 64 + lane]);
        const u32x4 w0 = kv0 ? kr0[mm] : u32x4{0, 0, 0, 0};
        const u32x4 w1 = kv1 ? kr1[mm] : u32x4{0, 0, 0, 0};
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, w0), k1 = __builtin_bit_cast(bf16x8, w1);
        s0[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qh, s0[mm & 1], 0, 0, 0);
        s1[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qh, s1[mm & 1], 0, 0, 0);
        s0[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, ql, s0[mm & 1], 0, 0, 0);
        s1[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, ql, s1[mm & 1], 0, 0, 0);
    }
    float sv0[4], sv1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sv0[i] = (tv0 + i < t_e) ? s0[0][i] + s0[1][i] : -INFINITY;
        sv1[i] = (tv1 + i < t_e) ? s1[0][i] + s1[1][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sv0[0], sv0[1]), fmaxf(sv0[2], sv0[3])), fmaxf(fmaxf(sv1[0], sv1[1]), fmaxf(sv1[2], sv1[3])));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mnew = fmaxf(m, mx);                // finite: subtile st0 has a valid key
    const float alpha = exp2f(m - mnew);
    float p0[4], p1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = exp2f(sv0[i] - mnew);
        p1[i] = exp2f(sv1[i] - mnew);
    }
    lsum = lsum * alpha + (((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3])));
    m = mnew;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float ai = shfl_f(alpha, 4 * gq + i);
#pragma unroll
        for (int nt = 0; nt < NKB; ++nt) O[nt][i] *= ai;
    }
    uint16_t ph0[4], pl0[4], ph1[4], pl1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ph0[i] = f32_to_bf16(p0[i]);
        pl0[i] = f32_to_bf16(p0[i] - bf16_to_f32(ph0[i]));
        ph1[i] = f32_to_bf16(p1[i]);
        pl1[i] = f32_to_bf16(p1[i] - bf16_to_f32(ph1[i]));
    }
    auto pk2 = [](uint16_t a, uint16_t b) { return (u32)a | ((u32)b << 16); };
    const bf16x8 ph = as_bf16x8(pk2(ph0[0], ph0[1]), pk2(ph0[2], ph0[3]), pk2(ph1[0], ph1[1]), pk2(ph1[2], ph1[3]));
    const bf16x8 pl = as_bf16x8(pk2(pl0[0], pl0[1]), pk2(pl0[2], pl0[3]), pk2(pl1[0], pl1[1]), pk2(pl1[2], pl1[3]));
    const int vv0 = t_e - tv0, vv1 = t_e - tv1;
    const u32 m00 = vv0 >= 2 ? 0xFFFFFFFFu : (vv0 == 1 ? 0x0000FFFFu : 0u);
    const u32 m01 = vv0 >= 4 ? 0xFFFFFFFFu : (vv0 == 3 ? 0x0000FFFFu : 0u);
    const u32 m10 = vv1 >= 2 ? 0xFFFFFFFFu : (vv1 == 1 ? 0x0000FFFFu : 0u);
    const u32 m11 = vv1 >= 4 ? 0xFFFFFFFFu : (vv1 == 3 ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt) {
        const bf16x8 v = as_bf16x8(vr0[nt].x & m00, vr0[nt].y & m01, vr1[nt].x & m10, vr1[nt].y & m11);
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, v, O[nt], 0, 0, 0);
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, O[nt], 0, 0, 0);
    }
}

// The q^T operand of head r of the item's group (hi and lo bf16 parts, dims in
// the K-row order of attn_sub), from this lane's 4 x NKB fp32 q values (dims
// 32(kb/2) + 8gq + 4(kb%2) + i), scaled by qscale (0 for lanes past the group).
template <int HD>
I4D_DEVINL void attn_q_operand(const f4 (&qv)[HD / 16], float qs, s4* qop) {
    constexpr int NKB = HD / 16;
    const int lane = i4d_tid() & 63;
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

// Each wave's running state (m and the row sum per head, O per head and dim)
// to its LDS area: wm[16], wl[16], wo[16][HD] per wave.
template <int HD, int NT>
I4D_DEVINL void attn_waves_to_lds(char* lds, float m, float lsum, const f4 (&O)[HD / 16]) {
    constexpr int NKB = HD / 16;
    const int tid = i4d_tid(), lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    float* wbase = (float*)lds + wave * (16 * HD + 32);
    float lt = lsum;
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    if (gq == 0) { wbase[r] = m; wbase[16 + r] = lt; }
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) wbase[32 + (4 * gq + i) * HD + 16 * nt + r] = O[nt][i];
}

// The waves' states combined per (head h < G, dim d): this split's partial
// (M, L, unnormalised O).  sink(h, d, M, L, acc) is called once per (h, d).
template <int HD, int NT, class Sink>
I4D_DEVINL void attn_combine_waves(const char* lds, int G, Sink& sink) {
    constexpr int NW = NT / 64;
    for (int idx = i4d_tid(); idx < G * HD; idx += NT) {
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
        sink(h, d, M, L, acc);
    }
}

// The whole item: optional round-0 registers already loaded (pre = true),
// compute, per-item partial, and the merge by the last split to arrive.
template <int HD, int NT, int NSW, bool PAGED = false>
I4D_DEVINL void attn_item(const AttnArgs& a, int item, char* lds, AttnRegs<HD, NSW>& R, bool pre) {
    constexpr int NW = NT / 64, NKB = HD / 16;
    const int tid = i4d_tid(), lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int G = a.hq / a.hkv;
    const AttnGeo g = attn_geo(a, item);
    const int nsub = g.nsub;

    // the subtile holding the new key gets the side-buffer values just before
    // it is used (in whichever round loads it: a line loaded earlier may be
    // stale); the other subtiles' loads are not waited for by these
    const int stp = (a.kvn != nullptr && g.kpos >= g.t_s && g.kpos < g.t_e) ? (g.kpos - g.t_s) / 16 : -1;
    // q first: its loads then only wait for themselves, not for the K/V stream
    // issued after them.  q^T operand (hi, lo) for head r of this group, dims
    // in the K-row order above, kept in LDS after the per-wave areas (every
    // wave uses the same operands).
    f4 qv[NKB];
    if (wave == 0) {
        const float* qrow = a.q + (size_t)(g.b * a.hq + g.j * G + min(r, G - 1)) * HD + 8 * gq;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qv[kb] = ld_g((const f4*)(qrow + 32 * (kb >> 1) + 4 * (kb & 1)));
    }
    const int nround = (nsub + NW * NSW - 1) / (NW * NSW);
    size_t poff[NSW];                                   // paged: pool offsets of the next round's subtiles
    if constexpr (PAGED) attn_page_offsets<HD, NT, NSW>(a, g, 0, poff);
    if (!pre) attn_load_round<HD, NT, NSW, PAGED>(a, g, 0, R, poff);
    if constexpr (PAGED) {
        if (nround > 1) attn_page_offsets<HD, NT, NSW>(a, g, 1, poff);
    }
    s4* qop = (s4*)(lds + NW * (16 * HD + 32) * 4);
    if (wave == 0) attn_q_operand<HD>(qv, (r < G) ? a.qscale : 0.f, qop);
    __syncthreads();

    float m = -INFINITY, lsum = 0.f;
    f4 O[NKB];
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt) O[nt] = f4{0.f, 0.f, 0.f, 0.f};

    // rounds of NSW subtiles per wave: round 0 is in R already
    for (int rnd = 0; rnd < nround; ++rnd) {
        if (rnd > 0) {
            attn_load_round<HD, NT, NSW, PAGED>(a, g, rnd, R, poff);
            if constexpr (PAGED) {
                if (rnd + 1 < nround) attn_page_offsets<HD, NT, NSW>(a, g, rnd + 1, poff);
            }
        }
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int st = (rnd * NSW + i) * NW + wave;
            if (st == stp) attn_patch_new<HD>(a, g, st, R.k[i], R.v[i]);
            if (st < nsub) attn_sub<HD>(g, st, R.k[i], R.v[i], qop, m, lsum, O);
        }
    }

    attn_waves_to_lds<HD, NT>(lds, m, lsum, O);
    __syncthreads();

    // combine the waves; write this split's partial (through to memory)
    const size_t hrow0 = (size_t)(g.b * a.hq + g.j * G);
    auto put = [&](int h, int d, float M, float L, float acc) {
        const size_t pidx = (hrow0 + h) * a.pstride + g.s;
        st_dev(a.po + pidx * HD + d, acc);
        if (d == 0) { st_dev(a.pm + pidx, M); st_dev(a.pl + pidx, L); }
    };
    attn_combine_waves<HD, NT>(lds, G, put);
    wait_stores();
    __syncthreads();

    // arrival: the last split of (b, j) merges
    int* last = (int*)lds;
    if (tid == 0) {
        int* c = a.cnt + g.b * a.hkv + g.j;
        const int old = __hip_atomic_fetch_add((I4D_GLOBAL int*)c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = (old == a.nsplit - 1);
        if (is_last) st_dev(c, 0);                  // ready for the next call
        last[0] = is_last;
    }
    __syncthreads();
    const bool merge = last[0] != 0;
    __syncthreads();
    if (merge) {
        // o[h][d] = sum_s w_s O_s[h][d] with w_s = 2^(m_s - M) / sum_s l_s 2^(m_s - M).
        // Threads own (head, 4 dims) slots; with more threads than slots each
        // slot's splits are cut into contiguous chunks summed in chunk order.
        // The first MB partial rows of every thread are requested before the
        // maxima, so the merge costs about one memory round trip.
        // LDS: 2*G*ns + 32 floats + NT float4 (at most 25 KB, inside the
        // per-wave area for every supported shape).
        constexpr int MB = NT >= 512 ? 16 : 32;
        const int ns = a.nsplit;
        const int slots = G * (HD / 4);
        const int chunks = max(1, NT / slots);
        float* sw = (float*)lds;                     // [G][ns] maxima, then weights
        float* sl = sw + G * ns;                     // [G][ns] sums
        float* hm = sl + G * ns;                     // [G] max, [G] 1 / L
        f4* part = (f4*)(lds + ((2 * G * ns + 32) * 4 + 15) / 16 * 16);   // [chunks][slots]
        const bool live = tid < slots * chunks;
        const int slot = live ? tid % slots : 0, chunk = live ? tid / slots : 0;
        const int h = slot / (HD / 4), d4 = slot - h * (HD / 4);
        const f4* src = (const f4*)(a.po + (hrow0 + h) * a.pstride * HD) + d4;
        const int per = (ns + chunks - 1) / chunks;
        const int s_lo = min(chunk * per, ns), s_hi = min(ns, s_lo + per);
        // Plain loads of the other splits' partials are safe only because no
        // workgroup reads these lines earlier in this launch, so the XCD's L2
        // cannot hold a stale copy: the writers stored them through to memory
        // and raised the counter after the stores completed.  Any read of
        // a.pm / a.pl / a.po before this point would break that and must then
        // use device-scope loads (ld_dev).
        f4 pv[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) pv[u] = ld_g(src + (size_t)min(s_lo + u, ns - 1) * (HD / 4));
        for (int idx = tid; idx < G * ns; idx += NT) {
            const int hh = idx / ns, ss = idx - hh * ns;
            const size_t pidx = (hrow0 + hh) * a.pstride + ss;
            sw[idx] = ld_g(a.pm + pidx);
            sl[idx] = ld_g(a.pl + pidx);
        }
        __syncthreads();
        // per-head maximum and sum, 32 threads per head (uniform trip count;
        // the shuffles stay inside each 32-lane group)
        for (int h0 = 0; h0 < G; h0 += NT / 32) {
            const int hh = h0 + (tid >> 5), lt = tid & 31;
            const bool ok = hh < G;
            float M = -INFINITY;
            if (ok)
                for (int ss = lt; ss < ns; ss += 32) M = fmaxf(M, sw[hh * ns + ss]);
            for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
            float L = 0.f;
            if (ok && M != -INFINITY)
                for (int ss = lt; ss < ns; ss += 32) L = fmaf(sl[hh * ns + ss], exp2f(sw[hh * ns + ss] - M), L);
            for (int o = 16; o >= 1; o >>= 1) L += shfl_xor_f(L, o);
            if (ok && lt == 0) { hm[hh] = M; hm[G + hh] = (L > 0.f) ? 1.0f / L : 0.f; }
        }
        __syncthreads();
        for (int idx = tid; idx < G * ns; idx += NT) {
            const int hh = idx / ns;
            const float M = hm[hh];
            sw[idx] = (M != -INFINITY) ? exp2f(sw[idx] - M) * hm[G + hh] : 0.f;
        }
        __syncthreads();
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = s_lo; s0 < s_hi; s0 += MB) {
            if (s0 > s_lo) {
#pragma unroll
                for (int u = 0; u < MB; ++u) pv[u] = ld_g(src + (size_t)min(s0 + u, ns - 1) * (HD / 4));
            }
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                if (s0 + u < s_hi) {
                    const float ws = sw[h * ns + s0 + u];
                    acc.x = fmaf(ws, pv[u].x, acc.x); acc.y = fmaf(ws, pv[u].y, acc.y);
                    acc.z = fmaf(ws, pv[u].z, acc.z); acc.w = fmaf(ws, pv[u].w, acc.w);
                }
            }
        }
        if (live) part[chunk * slots + slot] = acc;
        __syncthreads();
        for (int sl2 = tid; sl2 < slots; sl2 += NT) {
            f4 t = part[sl2];
            for (int c = 1; c < chunks; ++c) t += part[c * slots + sl2];
            const int hh = sl2 / (HD / 4), dd = sl2 - hh * (HD / 4);
            float* dst = a.o + (hrow0 + hh) * HD + 4 * dd;
            st_dev(dst, t.x); st_dev(dst + 1, t.y); st_dev(dst + 2, t.z); st_dev(dst + 3, t.w);
        }
    }
    __syncthreads();       // LDS is reused by the next item
}
