// Prompt prefill on the matrix cores (gfx950, wave64).
//
// Prefill gives every prompt token what decoding the tokens one after another
// would (Primer 1.2, the prefill/decode split), but it reads each weight once
// per tile of prompt tokens instead of once per token: the int4 projections
// become GEMMs with the prompt as the wide dimension, and attention becomes a
// causal attention tiled over the prompt (Roofline reply, section 四:
// FlashAttention-style tiling keeps the score matrix on chip).
//
// GEMM.  out[t][row] = sum_k x[t][k] w[row][k] for the T prompt tokens, with
// v_mfma_f32_16x16x32_f16: A = staged activations (16 tokens x 32 inputs),
// B = int4 weights expanded to exact fp16 in registers (16 rows x 32 inputs),
// fp32 accumulation.  The activations are the staged fp16 rows of the batched
// decode path (k_mfma_stage: RMSNorm folded in, the unpack's input order, odd
// inputs pre-divided by 16, one power of two per token for fp16 range), so
// the integer unpack and the group-scale handling are the ones of that path.
//
// Tile.  A workgroup (4 waves) owns BM tokens x 256 weight rows; each wave
// owns 4 row tiles of 16 (the pair mapping of the decode kernels: lanes r and
// r ^ 8 of a tile hold the two rows of a pair) for all BM tokens, i.e. 4 BM / 16
// accumulator tiles.  BM = 64, two waves per SIMD (the kernels are built
// for that register budget).  BM = 128 at one wave per SIMD, where each
// expanded weight feeds twice the MFMAs, measured slower: the second wave's
// latency hiding is worth more than the halved expansion.  The K axis is walked in steps of 128 inputs (one group
// of 128 or half a group of 256): per step a wave expands its 4 x 64 bytes of
// codes per lane-row into B operands once and runs 4 (tokens) x 4 (rows) x 4
// (32-input slices) MFMAs per activation plane; each (token tile, row tile)
// accumulates a step into a fresh tile that is then scaled by the row's
// group scale and added to the running sum (sum_k (c_k - 8) s x_k = s C).
//
// Activations reach LDS with gfx950's 16-byte global-to-LDS loads (no
// register staging): one wave instruction fills 1 KB, four token rows of one
// step.  Rows are not padded; instead the 16-byte piece p of token row t is
// stored at piece p ^ (t & 15), so that the 16 lanes of an MFMA operand read
// (different rows, same piece) hit 16 different bank groups.  Two LDS buffers:
// step s + 1 is loaded while step s is consumed, and one barrier per step
// (after waiting for the step's loads) hands the buffers over.  Weights go
// straight to registers, one step ahead.
//
// Grid.  Workgroups are numbered so that consecutive tiles of the same weight
// rows (all token tiles of one row block) land on the same XCD (the hardware
// deals workgroups to the 8 XCDs in turn): the row block's codes are then
// fetched from HBM once per XCD and served from its L2 to the other token
// tiles.  When the tiles alone do not fill the chip, the K axis is split and
// the partial sums are added by a separate pass in split order.
//
// Attention.  One wave per (query head, block of 16 prompt tokens): the
// columns of its score tile are the 16 tokens, so each key tile loaded feeds
// 16 queries (decode's attention puts the G heads of one token there).  Keys
// run from slot 0 up to the block's last position in 16-key tiles, two per
// online-softmax step (the 16x16x32 bf16 mapping of the decode attention);
// key k is masked for token t when k > pos(t) (causal), and K/V rows past the
// block's last position are zeroed (their slots may hold anything).  The
// first step always holds key 0, which every token attends, so every
// column's running maximum is finite from the first step on.
#pragma once
#include "attention.h"
#include "common.h"
#include "gemv.h"
#include "mfma.h"

constexpr int PF_NT = 256;                          // threads per GEMM workgroup
#ifndef I4D_PF_BM_WIDE
#define I4D_PF_BM_WIDE 64
#endif
constexpr int PF_BM_MAX = 128;                      // staged rows are padded to a multiple of this
constexpr int PF_BM_QKV = 64;                       // tokens per workgroup tile: q/k/v (two activation planes)
constexpr int PF_BM_WIDE = I4D_PF_BM_WIDE;          // gate/up
#ifndef I4D_PF_BM_ROWS
#define I4D_PF_BM_ROWS 64
#endif
constexpr int PF_BM_ROWS = I4D_PF_BM_ROWS;          // Wo and W_down (adjacent-row GEMMs + residual)
constexpr int PF_WT = 4;                            // 16-row tiles per wave
constexpr int PF_BN = (PF_NT / 64) * PF_WT * 16;    // weight rows per workgroup (256)
constexpr int PF_PAIRS = PF_BN / 2;                 // pairs per workgroup
// one step of one activation plane in LDS, and the two buffers of all planes
template <int BM> __host__ __device__ constexpr int pf_plane_bytes() { return BM * 256; }
template <int PREC, int BM> __host__ __device__ constexpr int pf_lds_bytes() { return 2 * PREC * pf_plane_bytes<BM>(); }

struct PfTask {
    GemvTask t;              // matrices and pair mapping (int4, groups of 128 or 256)
    const uint32_t* xs;      // staged activations [PREC][sp][K/2] (uint32 = two fp16)
    const float* xscale;     // [sp] power of two that multiplies token t's results
    float* part;             // K split: partial sums [ks][ntok][rows]
    int sp;                  // staged rows per plane (tokens rounded up to PF_BM_MAX)
    int ntok;                // prompt tokens
    int nsteps;              // K / 128
    int gshift;              // log2(group / 128)
    int mtiles, ntiles;      // token tiles, row blocks
    int ks, spk;             // K splits, steps per split
    int rows;                // output rows of the partial sums (K split)
    int nlo;                 // row blocks 0 .. nlo - 1 run on the value plane alone (q/k/v: the q rows); 0: none
};

// Tile of this workgroup: the hardware sends workgroup i to XCD i % 8, so
// XCD x gets a contiguous range of tile indices, token tile fastest.
I4D_DEVINL void pf_tile(const PfTask& g, int& mt, int& nt, int& kss) {
    const int nwg = g.mtiles * g.ntiles * g.ks;
    const int id = blockIdx.x, x = id & 7, local = id >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int w = x * per + min(x, rem) + local;
    mt = w % g.mtiles;
    const int rest = w / g.mtiles;
    const int u = rest % g.ntiles, N = g.ntiles, nh = N - g.nlo;
    kss = rest / g.ntiles;
    nt = u;
    if (g.nlo > 0 && nh > 0) {
        // one-plane blocks cost about half a two-plane block: deal the nh
        // two-plane blocks evenly over the block order, each first in its
        // run, so that every XCD gets its share and starts them first
        const int c0 = (u * nh + N - 1) / N, c1 = ((u + 1) * nh + N - 1) / N;
        nt = c0 < c1 ? g.nlo + c0 : u - c0;
    }
}

typedef __attribute__((address_space(3))) void* lds_vptr;

// wait for every outstanding load (global-to-LDS included) and LDS access of
// this wave, then the workgroup barrier
I4D_DEVINL void pf_sync() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// BM tokens per workgroup tile (BM / 16 token tiles per wave)
template <int KND, int PREC, int BM, class Epi>
I4D_DEVINL void pf_gemm(const PfTask& g, char* lds, Epi& epi) {
    constexpr int MT = BM / 16, RPW = BM / (PF_NT / 64), PLANE_B = pf_plane_bytes<BM>();
    int mt, nt, kss;
    pf_tile(g, mt, nt, kss);
    const int tid = i4d_tid(), wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    const int tok0 = mt * BM;
    const int s0 = kss * g.spk, s1 = min(g.nsteps, s0 + g.spk);
    const size_t K2 = (size_t)(g.t.k >> 1);           // uint32 per staged row

    // this lane's weight row in each of the wave's tiles: codes from byte 16 q
    // of each 64-byte step, and the row's scales
    const uint8_t* wp[PF_WT];
    const uint16_t* sp[PF_WT];
#pragma unroll
    for (int i = 0; i < PF_WT; ++i) {
        const int T = nt * (PF_BN / 16) + wave * PF_WT + i;
        const RowPtrs rp = resolve_pair<FMT_INT4_FAST, KND>(g.t, min(8 * T + (r & 7), g.t.total_pairs - 1));
        wp[i] = (r < 8 ? rp.pa : rp.pb) + 16 * q;
        sp[i] = r < 8 ? rp.sa : rp.sb;
    }

    // step s of the BM token rows into LDS buffer b: wave w fills rows
    // RPW w .. RPW w + RPW - 1, four rows (1 KB) per instruction; lane l writes
    // piece l & 15 of its row, which holds the row's piece (l & 15) ^ (row & 15)
    auto load_a = [&](int b, int s) {
#pragma unroll
        for (int p = 0; p < PREC; ++p)
#pragma unroll
            for (int i = 0; i < RPW / 4; ++i) {
                const int rl = 4 * i + (lane >> 4);
                const int row = RPW * wave + rl;               // the read side swizzles by row & 15
                const uint32_t* src = g.xs + ((size_t)p * g.sp + tok0 + row) * K2 + (size_t)s * 64 +
                                      (((lane & 15) ^ (row & 15)) << 2);
                char* dst = lds + (b * PREC + p) * PLANE_B + (RPW * wave + 4 * i) * 256;
                __builtin_amdgcn_global_load_lds((const I4D_GLOBAL void*)src, (lds_vptr)dst, 16, 0, 0);
            }
    };
    u32x4 wr[PF_WT];
    u32 scr[PF_WT];
    auto load_w = [&](int s) {
#pragma unroll
        for (int i = 0; i < PF_WT; ++i) {
            wr[i] = ld_g_nt((const u32x4*)(wp[i] + (size_t)s * 64));
            scr[i] = (u32)ld_g(sp[i] + (s >> g.gshift));
        }
    };

    f4 acc[MT][PF_WT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < PF_WT; ++i) acc[m][i] = f4{0.f, 0.f, 0.f, 0.f};

    load_a(0, s0);
    load_w(s0);
    pf_sync();
    for (int s = s0; s < s1; ++s) {
        const int b = (s - s0) & 1;
        // this step's codes -> B operands, then the next step's loads
        h8 bw[PF_WT][4];
        float sc[PF_WT];
#pragma unroll
        for (int i = 0; i < PF_WT; ++i) {
            bw[i][0] = unpack_b(wr[i].x);
            bw[i][1] = unpack_b(wr[i].y);
            bw[i][2] = unpack_b(wr[i].z);
            bw[i][3] = unpack_b(wr[i].w);
            sc[i] = __uint_as_float(scr[i] << 16);
        }
        if (s + 1 < s1) {
            load_a(b ^ 1, s + 1);
            load_w(s + 1);
        }
        const char* ab = lds + b * PREC * PLANE_B;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f4 cg[PF_WT];
#pragma unroll
            for (int i = 0; i < PF_WT; ++i) cg[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int p = 0; p < PREC; ++p) {
                    const h8 a = *(const h8*)(ab + p * PLANE_B + (16 * m + r) * 256 + (((4 * q + j) ^ r) << 4));
#pragma unroll
                    for (int i = 0; i < PF_WT; ++i) cg[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[i][j], cg[i], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < PF_WT; ++i) {
                acc[m][i].x = fmaf(sc[i], cg[i].x, acc[m][i].x);
                acc[m][i].y = fmaf(sc[i], cg[i].y, acc[m][i].y);
                acc[m][i].z = fmaf(sc[i], cg[i].z, acc[m][i].z);
                acc[m][i].w = fmaf(sc[i], cg[i].w, acc[m][i].w);
            }
        }
        pf_sync();
    }

    // lane (r, q) holds tokens 16 m + 4 q + e of tile row r
    if (g.ks == 1) {
#pragma unroll
        for (int i = 0; i < PF_WT; ++i) {
            const int pair = 8 * (nt * (PF_BN / 16) + wave * PF_WT + i) + r;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = acc[m][i][e];
                    const float o = shfl_xor_f(v, 8);
                    const int t = tok0 + 16 * m + 4 * q + e;
                    if (r < 8 && pair < g.t.total_pairs && t < g.ntok) {
                        const float xsc = ld_g(g.xscale + t);
                        epi(0, pair, t, v * xsc, o * xsc);
                    }
                }
        }
    } else {
        // K split (adjacent-row pairs only): raw sums to part[kss][t][row]
#pragma unroll
        for (int i = 0; i < PF_WT; ++i) {
            const int row = 2 * (8 * (nt * (PF_BN / 16) + wave * PF_WT + i) + (r & 7)) + (r >> 3);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = tok0 + 16 * m + 4 * q + e;
                    if (row < g.rows && t < g.ntok) st_g(g.part + ((size_t)kss * g.ntok + t) * g.rows + row, acc[m][i][e]);
                }
        }
    }
}

// y[t][row] = resid[t][row] + xscale[t] * (sum over splits k in order of part[k][t][row])
__global__ void __launch_bounds__(256) k_pf_reduce(const float* part, int ks, int ntok, int rows, const float* xscale,
                                                   const float* resid, float* y) {
    const size_t n = (size_t)ntok * rows;
    for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (size_t)gridDim.x * 256) {
        float v = 0.f;
        for (int k = 0; k < ks; ++k) v += ld_g(part + (size_t)k * n + idx);
        const int t = (int)(idx / rows);
        st_g(y + idx, (resid ? ld_g(resid + idx) : 0.f) + v * ld_g(xscale + t));
    }
}

// prompt positions pos0 .. pos0 + n - 1
__global__ void __launch_bounds__(256) k_pf_positions(int* pos, int n, int pos0) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < n) pos[t] = pos0 + t;
}

// ---------------------------------------------------------------- attention
struct PfAttnArgs {
    const float* q;          // [T][Hq][hd] fp32 (RoPE applied)
    const uint16_t* kc;      // the sequence's K cache (row 0 of the layout, or the page pool)
    const uint16_t* vc;      // the sequence's V cache
    float* o;                // [T][Hq][hd] fp32
    int ntok, pos0, cap, hq, hkv, nqb;
    float qscale;            // log2(e) / sqrt(hd)
    KvMap pg;
    int* status;
};

// K rows (key 16 st + r, dims 32 mm + 8 g .. + 8) and V (dims 16 nt + r, keys
// 16 st + 4 g .. + 3) of tile st of KV head j
template <int HD>
I4D_DEVINL void pf_load_tile(const PfAttnArgs& a, int j, int st, u32x4 (&kr)[HD / 32], u32x2 (&vr)[HD / 16]) {
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    bool bad = false;
    const size_t tile = kv_tile_off(a.pg, a.cap, a.hkv, HD, 0, j, st, bad);
    if (bad && lane == 0 && a.status) raise_status(a.status, I4D_DEV_BAD_PAGE);
    const uint16_t* kp = a.kc + tile + r * 32 + 8 * gq;
#pragma unroll
    for (int mm = 0; mm < HD / 32; ++mm) kr[mm] = ld_g((const u32x4*)(kp + 512 * mm));
    const uint16_t* vp = a.vc + tile + r * 16 + 4 * gq;
#pragma unroll
    for (int nt = 0; nt < HD / 16; ++nt) vr[nt] = ld_g((const u32x2*)(vp + 256 * nt));
}

// One online-softmax step over key tiles st0 and st0 + 1 for 16 query columns
// (lane (r, g): column r).  pcol: this lane's column position (keys <= pcol
// are attended); kend: one past the last key whose K/V slot is written.
template <int HD>
I4D_DEVINL void pf_attn_step(int st0, int pcol, int kend, const u32x4 (&kr0)[HD / 32], const u32x2 (&vr0)[HD / 16],
                             const u32x4 (&kr1)[HD / 32], const u32x2 (&vr1)[HD / 16], const u32x4 (&q32)[HD / 16],
                             float& m, float& lsum, f4 (&O)[HD / 16]) {
    constexpr int NKB = HD / 16, NMM = HD / 32;
    const int lane = i4d_tid() & 63, r = lane & 15, gq = lane >> 4;
    const int k00 = 16 * st0, k01 = k00 + 16;
    const bool kv0 = k00 + r < kend, kv1 = k01 + r < kend;
    f4 s0[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    f4 s1[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm) {
        const bf16x8 qh = __builtin_bit_cast(bf16x8, q32[2 * mm]);
        const bf16x8 ql = __builtin_bit_cast(bf16x8, q32[2 * mm + 1]);
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, kv0 ? kr0[mm] : u32x4{0, 0, 0, 0});
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, kv1 ? kr1[mm] : u32x4{0, 0, 0, 0});
        s0[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qh, s0[mm & 1], 0, 0, 0);
        s1[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qh, s1[mm & 1], 0, 0, 0);
        s0[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, ql, s0[mm & 1], 0, 0, 0);
        s1[mm & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, ql, s1[mm & 1], 0, 0, 0);
    }
    // lane (r, g) holds the scores of keys 4 g + i of both tiles for column r
    const int kv = k00 + 4 * gq, kw = k01 + 4 * gq;
    float sv0[4], sv1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sv0[i] = (kv + i <= pcol) ? s0[0][i] + s0[1][i] : -INFINITY;
        sv1[i] = (kw + i <= pcol) ? s1[0][i] + s1[1][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sv0[0], sv0[1]), fmaxf(sv0[2], sv0[3])), fmaxf(fmaxf(sv1[0], sv1[1]), fmaxf(sv1[2], sv1[3])));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mnew = fmaxf(m, mx);                // finite from the first step on (key 0)
    const float alpha = exp2f(m - mnew);
    float p0[4], p1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = exp2f(sv0[i] - mnew);
        p1[i] = exp2f(sv1[i] - mnew);
    }
    lsum = lsum * alpha + (((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3])));
    m = mnew;
    // O rows are columns 4 g + i: rescale each by its column's alpha
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
    auto pk2 = [](uint16_t x, uint16_t y) { return (u32)x | ((u32)y << 16); };
    const bf16x8 ph = as_bf16x8(pk2(ph0[0], ph0[1]), pk2(ph0[2], ph0[3]), pk2(ph1[0], ph1[1]), pk2(ph1[2], ph1[3]));
    const bf16x8 pl = as_bf16x8(pk2(pl0[0], pl0[1]), pk2(pl0[2], pl0[3]), pk2(pl1[0], pl1[1]), pk2(pl1[2], pl1[3]));
    // V keys past kend are zeroed (P is zero there, but the slot may hold a non-finite value)
    const int vv0 = kend - kv, vv1 = kend - kw;
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

// One wave per (query head h, 16-token block); the heaviest blocks (the last
// of the prompt, which attend the most keys) are numbered first.
template <int HD>
__global__ void __launch_bounds__(256) k_pf_attn(PfAttnArgs a) {
    constexpr int NKB = HD / 16, NMM = HD / 32;
    const int tid = i4d_tid(), lane = tid & 63, r = lane & 15, gq = lane >> 4;
    const int gw = blockIdx.x * 4 + (tid >> 6);
    if (gw >= a.hq * a.nqb) return;
    const int h = gw % a.hq, qb = a.nqb - 1 - gw / a.hq;
    const int j = h / (a.hq / a.hkv);
    const int t0 = 16 * qb;
    const int live = min(16, a.ntok - t0);
    const int tcol = t0 + min(r, live - 1);          // columns past the prompt repeat its last token
    const int pcol = a.pos0 + tcol;
    const int kend = a.pos0 + t0 + live;             // keys 0 .. kend - 1 are written

    // q^T operand: lane (r, g) holds dims 32 mm + 8 g .. + 7 of column r, as
    // high and low bf16 parts of q * qscale
    u32x4 q32[NKB];
    const float* qp = a.q + ((size_t)tcol * a.hq + h) * HD + 8 * gq;
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm) {
        const f4 x0 = ld_g((const f4*)(qp + 32 * mm)), x1 = ld_g((const f4*)(qp + 32 * mm + 4));
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint16_t hv[8], lv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = xv[e] * a.qscale;
            hv[e] = f32_to_bf16(v);
            lv[e] = f32_to_bf16(v - bf16_to_f32(hv[e]));
        }
        q32[2 * mm] = u32x4{(u32)hv[0] | ((u32)hv[1] << 16), (u32)hv[2] | ((u32)hv[3] << 16), (u32)hv[4] | ((u32)hv[5] << 16),
                            (u32)hv[6] | ((u32)hv[7] << 16)};
        q32[2 * mm + 1] = u32x4{(u32)lv[0] | ((u32)lv[1] << 16), (u32)lv[2] | ((u32)lv[3] << 16),
                                (u32)lv[4] | ((u32)lv[5] << 16), (u32)lv[6] | ((u32)lv[7] << 16)};
    }

    float m = -INFINITY, lsum = 0.f;
    f4 O[NKB];
#pragma unroll
    for (int nt = 0; nt < NKB; ++nt) O[nt] = f4{0.f, 0.f, 0.f, 0.f};
    const int ntiles = (kend + 15) >> 4;
    for (int st = 0; st < ntiles; st += 2) {
        u32x4 k0[NMM], k1[NMM];
        u32x2 v0[NKB], v1[NKB];
        pf_load_tile<HD>(a, j, st, k0, v0);
        pf_load_tile<HD>(a, j, min(st + 1, ntiles - 1), k1, v1);     // a tile past the keys: all masked
        pf_attn_step<HD>(st, pcol, kend, k0, v0, k1, v1, q32, m, lsum, O);
    }

    // O / l, column 4 g + i of lane (r, g) holding dims 16 nt + r
    float lt = lsum;
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 4 * gq + i;
        const float inv = 1.0f / shfl_f(lt, c);
        if (c < live) {
            float* op = a.o + ((size_t)(t0 + c) * a.hq + h) * HD + r;
#pragma unroll
            for (int nt = 0; nt < NKB; ++nt) st_g(op + 16 * nt, O[nt][i] * inv);
        }
    }
}
