// fa_fwd_mfma16.hpp — fused attention forward for bf16 / fp16 inputs on gfx950.
//
// The algorithm is the query-outer, key-inner online-softmax recurrence of the
// course page "05_flash_attention.py" (flash_attention_forward): per query tile
// m = -inf, l = 0, O~ = 0; for each key/value tile, left to right:
//     S = Q_i K_j^T * scale,  m_new = max(m, rowmax S),  P = exp(S - m_new),
//     alpha = exp(m - m_new), l = alpha l + rowsum P, O~ = alpha O~ + P V_j;
// at the end O = O~ / l and L = m + log l.  The unnormalised O~ is rescaled by
// exp(m_old - m_new) alone, as in the "Flash Attention" blog page's (+) operator
// on (m, d, o~).  Key tiles wholly in the causal future are skipped and only
// tiles that straddle the diagonal (or the ragged end of the keys) are masked
// (course page, causal branch of flash_attention_forward).
//
// gfx950 mapping (designed for CDNA4, not taken from the pages' NVIDIA design):
//   * wave w owns query rows [32w, 32w+32) of its workgroup's tile; for d = 128 a
//     workgroup is 8 waves (256 rows) and fills a CU alone, for d = 64 it is 4 waves
//     (128 rows) and two share a CU: either way each SIMD interleaves two waves, and
//     each staged K/V tile serves as many query rows as fit;
//   * key groups (d = 64, grids of at most 256 of those 128-row workgroups, which
//     would leave CUs idle and run one wave per SIMD through all the key tiles): a
//     workgroup is 2 query waves (64 rows) times 4 key groups, group g takes key
//     tiles g, g + 4, ... with K/V buffers of its own, so each SIMD interleaves two
//     waves and each wave's chain of tiles is a quarter as long; at the end the
//     groups' (m, l, O~) states are folded with the blog page's (+) operator through
//     LDS, and group 0 writes the result;
//   * both contractions on v_mfma_f32_32x32x16_{bf16,f16}; S is computed
//     transposed, S^T = K Q^T, so each lane owns ONE query (lane % 32) and 16 of
//     the 32 keys of a 32-key block: the row max needs one exchange between the
//     wave halves, the row sum none until the epilogue;
//   * O is accumulated transposed, O^T = V^T P^T: alpha is a per-lane scalar and P
//     is the MFMA B operand straight from the S registers (rounded to T);
//   * K tiles go global -> LDS by DMA (buffer_load ... lds, 16 B per lane) into
//     rows padded by 16 B, so that the K reads (ds_read_b128) of 16 consecutive
//     rows hit 64 distinct banks and every operand address is one base register
//     plus an immediate; a DMA block is 1 KB of consecutive LDS and lanes that land
//     on padding are masked off;
//   * V goes to LDS by DMA as well, rows as stored (padded to 2D + 32 bytes), and
//     the A operand of O^T = V^T P^T comes from gfx950's transposing LDS read
//     (tr_operand in fa_tiles.hpp), its keys in the order P has in registers; the
//     DMA is issued from inline assembly so that the compiler does not make those
//     reads wait for every DMA in flight, and each step's barrier waits for it;
//   * every buffer access goes through a buffer resource bounded by the head's
//     remaining rows, so rows past Nk read as zero without a branch;
//   * software pipeline: while the softmax of tile j and the P.V MFMAs of tile j
//     run, the S MFMAs of tile j+1 are issued; K and V have separate double
//     buffers with the next loads issued one tile ahead; one barrier per tile;
//   * exp is exp2 with scale*log2(e) folded into one FMA; the running-max reference
//     moves (with the O~ rescale) on a new row maximum while the row's sum is small,
//     and once it is large only when a key would weigh more than 1/5 of the row
//     (P never exceeds 2^8); L takes the fp32 row sum of P, O the row sum of the
//     rounded P it was built from (see update_max).
#pragma once

#include <type_traits>

#include "fa_philox.hpp"
#include "fa_tiles.hpp"

namespace fa {

template <int D, int KG = 1>
struct Tile16 {
    // d = 128: 8 waves (256 query rows) share each staged K/V tile, one workgroup
    // per CU (2 waves per SIMD); d = 64: 4 waves (128 rows), two workgroups per CU,
    // so that the small-d grids still cover the chip.  KG > 1 (d = 64, for grids too
    // small to give every CU a workgroup): 2 query waves (64 rows) times KG key groups;
    // group g takes key tiles g, g + KG, g + 2 KG, ... with K/V buffers of its own,
    // and the groups' states are merged by the (+) operator at the end.
    static constexpr int NQW = D == 128 ? 8 : (KG == 1 ? 4 : 2);  // query waves
    static constexpr int NW = NQW * KG;          // waves per workgroup
    static constexpr int BR = 32 * NQW;          // query rows per workgroup
    static constexpr int BC = 64;                // keys per K/V tile
    static constexpr int NT = 64 * NW;           // threads per workgroup
    static constexpr int GT = 64 * NQW;          // threads of one key group
    static constexpr int ROWB = D * 2;           // bytes per K/V row in memory
    static constexpr int KSTR = ROWB + 16;       // K row stride in LDS
    // V rows, read only transposed: with 2D + 32 bytes the 4 rows of a half-wave's
    // transposing read meet at most 2-way in the banks (2D + 64 would avoid that and
    // not fit the four key groups' buffers)
    static constexpr int VSTR = ROWB + 32;
    static constexpr int KT = BC * KSTR;         // bytes of one K tile in LDS
    static constexpr int VT = BC * VSTR;         // bytes of one V tile in LDS
    static constexpr int KNB = KT / 1024;        // 1-KB DMA blocks per K tile
    static constexpr int KPW = (KNB + NQW - 1) / NQW;  // K blocks per wave (at most)
    static constexpr int VNB = VT / 1024;        // 1-KB DMA blocks per V tile
    static constexpr int VPW = (VNB + NQW - 1) / NQW;
    static constexpr int DC = D / 16;            // 16-wide d chunks of the S contraction
    static constexpr int DB = D / 32;            // 32-wide d blocks of O
    static constexpr int GR = 2 * KT + 2 * VT;   // one key group's K[2], V[2]
    static constexpr int SUMS = KG * GR;         // per thread: completed row-sum blocks
    static constexpr int LDS = SUMS + 8 * NT;    // the groups' buffers, sums
    static constexpr int K0 = 0, K1 = KT, V0 = 2 * KT, V1 = 2 * KT + VT;  // in a group's
    // epilogue: a wave's 32 rows of O (2D bytes each) or of 64 fp32 partial columns
    // (256 bytes), staged in LDS with 16 bytes of padding
    static constexpr int OSTR = (2 * D > 256 ? 2 * D : 256) + 16;
    static_assert(NQW * 32 * OSTR <= SUMS, "the epilogue's rows must fit the tile buffers");
    static_assert(KT % 1024 == 0 && VT % 1024 == 0, "tiles must be whole DMA blocks");
    // KG > 1: the state one wave of group g > 0 hands to group 0 (per lane: O^T
    // registers, this half's two row sums, the reference), past the epilogue's rows
    static constexpr int XSTR = 4 * (16 * DB + 4);   // bytes per lane
    static constexpr int XOFF = (NQW * 32 * OSTR + 1023) / 1024 * 1024;
    static_assert(KG == 1 || XOFF + (KG - 1) * NQW * 64 * XSTR <= SUMS,
                  "the merge's states must fit the tile buffers");
};

template <typename T, int D, bool CAUSAL, bool SPLIT, bool DROP = false, bool MASK = false,
          int KG = 1>
__global__ __launch_bounds__((Tile16<D, KG>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_mfma16_kernel(const FwdParams<T> prm)
{
    static_assert(KG == 1 || (D == 64 && !SPLIT && !DROP && !MASK),
                  "key groups serve the plain d = 64 forward");
    using P = Tile16<D, KG>;
    using M = Mfma16<T>;
    using vec = typename M::vec;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const char* const sm = smem;
    const int Nq = prm.Nq, Nk = prm.Nk, n_qtiles = prm.n_qtiles;
    const float c2 = prm.c2;

    // ---- which (batch*head, key split, query tile) this workgroup owns; the
    // query tiles of one (head, split) are consecutive, so they share an XCD's L2
    const WorkItem wi = work_item((int)blockIdx.x, (int)gridDim.x, n_qtiles, CAUSAL && !SPLIT);
    const int rest = wi.head;
    const int qt = CAUSAL ? n_qtiles - 1 - wi.rank : wi.rank;  // longest rows (most key tiles) first
    const int split = SPLIT ? rest % prm.n_splits : 0;
    const int bh = SPLIT ? rest / prm.n_splits : rest;
    const int q0 = qt * P::BR;

    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6;
    const int qw = KG == 1 ? wave : wave % P::NQW;  // query wave: rows 32 qw .. of the tile
    const int grp = KG == 1 ? 0 : wave / P::NQW;    // key group: tiles grp, grp + KG, ...
    const int gbase = grp * P::GR;  // the group's K / V^T buffers
    const int lane = tid & 63;
    const int ql = lane & 31;  // query column of this lane in the accumulators
    const int hh = lane >> 5;  // wave half
    const int qw0 = q0 + qw * 32;
    const int my_q = qw0 + ql;

    // ---- key range: keys [kbeg, kbeg + Nks) of the head (all of them unless split);
    // key tiles and positions below are relative to kbeg, so a query's causal limit
    // is its index minus kbeg
    const int kbeg = SPLIT ? split * prm.split_tiles * P::BC : 0;
    const int Nks = SPLIT ? min(Nk - kbeg, prm.split_tiles * P::BC) : Nk;
    const int qkw0 = qw0 - kbeg;   // first query of the wave, in key positions
    const int my_qk = my_q - kbeg;

    const T* Qh = prm.q + (size_t)bh * Nq * D;
    const T* Kh = prm.k + ((size_t)bh * Nk + kbeg) * D;
    const T* Vh = prm.v + ((size_t)bh * Nk + kbeg) * D;

    // ---- key tiles: the workgroup stages nkt of them; this wave computes n_w
    // (a query before the range sees none of its keys)
    int nkt = (Nks + P::BC - 1) / P::BC;
    if (CAUSAL) {
        const int last = min(q0 + P::BR, Nq) - 1 - kbeg;
        nkt = last < 0 ? 0 : min(nkt, last / P::BC + 1);
    }
    const bool wave_active = qw0 < Nq;
    int n_w = wave_active ? nkt : 0;
    if (CAUSAL && wave_active) {
        const int last = min(qw0 + 31, Nq - 1) - kbeg;
        n_w = last < 0 ? 0 : min(nkt, last / P::BC + 1);
    }
    // the key group's share: local tile i is tile grp + KG i; ni_g of the workgroup's
    // tiles are staged by the group, this wave computes the first ni_w of them, and
    // every wave runs ni steps (the most any group has), so all pass the same barriers
    auto share = [&](int n) { return n > grp ? (n - grp + KG - 1) / KG : 0; };
    const int ni = (nkt + KG - 1) / KG;
    const int ni_g = share(nkt);
    const int ni_w = share(n_w);
    auto tile_of = [&](int i) { return grp + KG * i; };

    // ---- K staging by DMA: per-lane source offsets of this wave's blocks (fixed)
    int ksrc[P::KPW];
#pragma unroll
    for (int i = 0; i < P::KPW; ++i)
        ksrc[i] = dma_src<D>(qw + P::NQW * i, lane, P::KSTR);
    int vsrc[P::VPW];
#pragma unroll
    for (int i = 0; i < P::VPW; ++i)
        vsrc[i] = dma_src<D>(qw + P::NQW * i, lane, P::VSTR);
    auto stage_k = [&](int tile, int lds_off) {
        stage_tile_asm<D, P::KNB, P::KPW, P::NQW>(Kh, tile, Nks, smem + gbase + lds_off, qw, ksrc);
    };
    auto stage_v = [&](int tile, int lds_off) {
        stage_tile_asm<D, P::VNB, P::VPW, P::NQW>(Vh, tile, Nks, smem + gbase + lds_off, qw, vsrc);
    };
    // the step's barrier: this wave's DMA has landed (and its LDS reads are done),
    // then the workgroup barrier publishes the group's tiles
    auto dma_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        wg_barrier();
    };

    // ---- operand addresses inside a K / V tile: one base each, the rest immediates
    // K (A operand of S^T): lane reads K[32kb + ql][16c + 8hh .. +8] at
    // kbase + 32c + 32kb*KSTR.
    const int kbase = ql * P::KSTR + hh * 16;
    // V^T (A operand of O^T, read transposed from the V rows, tr_operand): lane
    // (h = lane / 32, g = (lane / 16) % 2, j = lane % 16) addresses row 4h + j / 4 at
    // dims 16g + 4 (j % 4), plus 16cc rows and 32db dims.
    const int tbase = (4 * hh + ((lane >> 2) & 3)) * P::VSTR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    // ---- caller mask: this lane's row of the head's mask slice; the words of tile t
    // sit in slot t % 2, loaded two tiles ahead of the S MFMAs that need them
    static_assert(!(MASK && SPLIT), "the masked forward is not split");
    const __amdgpu_buffer_rsrc_t mrs = mask_rsrc(MASK ? mask_slice(prm, bh) : nullptr, q0, P::BR, Nq,
                                                 MASK ? prm.mask_w : 0);
    int mrow_off = 0;
    uint32_t mwd[2][2] = {{0u, 0u}, {0u, 0u}};
    if (MASK)
        mrow_off = (my_q - q0) * prm.mask_w * 4;
    auto load_mask = [&](int t, int slot) {
        mwd[slot][0] = __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * t, 0, 0);
        mwd[slot][1] = __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * t + 4, 0, 0);
    };

    // ---- prologue: the group's tiles 0 and 1 in flight, Q fragment into registers
    if (MASK && 0 < ni_w)
        load_mask(tile_of(0), 0);
    if (MASK && 1 < ni_w)
        load_mask(tile_of(1), 1);
    if (0 < ni_g) {
        stage_k(tile_of(0), P::K0);
        stage_v(tile_of(0), P::V0);
    }
    if (1 < ni_g) {
        stage_k(tile_of(1), P::K1);
        stage_v(tile_of(1), P::V1);
    }
    // Q (B operand of S^T = K Q^T): lane supplies Q[my_q][16c + 8hh .. +8]
    vec qf[P::DC];
#pragma unroll
    for (int c = 0; c < P::DC; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (my_q < Nq)
            raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + 16 * c + 8 * hh);
        qf[c] = __builtin_bit_cast(vec, raw);
    }

    // S^T of one key tile from the K buffer at byte offset kb_off
    auto scores = [&](int kb_off, f32x16* s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            s[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < P::DC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const vec a = *reinterpret_cast<const vec*>(sm + kb_off + kbase + 32 * c + kb * 32 * P::KSTR);
                s[kb] = M::mma(a, qf[c], s[kb]);
            }
    };

    // ---- running state: base-2 reference max m2, this half's partial sum l, O^T
    f32x16 o[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        o[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = neg_inf();
    float l = 0.f;   // this half's sum of the fp32 P (for L), current block of tiles
    float lr = 0.f;  // this half's sum of the rounded P (for the normalisation of O), same
    // The row sums run per block of kSumBlock key tiles and are folded into this
    // thread's LDS slot (l, lr of the completed blocks) when a block ends: a sequential
    // fp32 sum over T tiles can drift by up to about T 2^-24 of its value (when the
    // tile sums are alike), blocks bound the drift by about (kSumBlock + T / kSumBlock)
    // 2^-24.  The slot is in LDS because the dropout instantiations have no register
    // to spare; it is touched once per block and on the rare rescale only.
    float* const done = reinterpret_cast<float*>(smem + P::SUMS) + 2 * tid;
    done[0] = 0.f;
    done[1] = 0.f;

    // Mask tile j: keys key0 + 4hh + off (off = 32kb + 8(r/4) + r%4) past the end of
    // the keys or (causal) after the query become -inf.  Only a wave's last tile can
    // need it: the wave's first query qw0 is a multiple of 32 and its last tile is
    // the one holding key min(qw0 + 31, Nq - 1) (or the last key), so every earlier
    // 64-key tile ends before qw0; the ragged end of the keys is the last tile.
    auto mask_tile = [&](int j, f32x16* s) {
        const int key0 = j * P::BC;
        const int last = CAUSAL ? min(Nks - 1, my_qk) : Nks - 1;
        const int lim = last - key0 - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                if (off > lim)
                    s[kb][r] = neg_inf();
            }
    };
    auto needs_mask = [&](int j) {
        const int key0 = j * P::BC;
        return (key0 + P::BC > Nks) || (CAUSAL && key0 + P::BC - 1 > qkw0);
    };

    // Running-max update with a reference that moves only when it matters: m2 (and
    // with it O~, l, lr, rescaled by alpha = 2^(m2 - m_new)) moves to the rows' maxima
    // when some lane of the wave sees its half of a row exceed m2 + g, where
    // g = clamp(e - kShift, 0, kSlack) and e is the binary exponent of a lower bound
    // of the row's running sum (l >= 2^(e-1)): this half's sum over the current block
    // of tiles, from an earlier tile (sums only grow between moves).  A key that does
    // not move the reference has P <= 2^g <= l / 4: it weighs at most 1/5 of its row,
    // and P <= 2^kSlack.  A key that does gets P = 1 exactly, as in the pages'
    // recurrence (which moves on every new maximum), so the weight of a row's dominant
    // key is not rounded; while l is small (peaked rows, the first tiles of a row)
    // every new maximum moves it, and once l is large the 32-multiply rescale is rare.
    // The halves' maxima are exchanged only on a move: m2 is the same in both halves
    // of a row because it is only ever set from the whole row's max.  Any reference
    // gives the same softmax: L = m2 + log2(sum P) uses the fp32 sum, and O is divided
    // by the sum of the SAME rounded P that went into the P.V MFMAs.  thr2 = m2 + g:
    // g = 0 after a move, recomputed after every second tile's sums.
    constexpr float kSlack = 8.0f;
    constexpr int kShift = 3;
    float thr2 = neg_inf();
    auto tile_max = [&](const f32x16* s) {
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[kb][r]);
        return mx;
    };
    auto update_max = [&](float mx) {
        const float mh = mx * c2;  // c2 > 0: max commutes with the scale
        if (__builtin_amdgcn_ballot_w64(mh > thr2) != 0) {
            const float m_new = fmaxf(m2, fa::half_max(mh));
            // 0 on a row's first visible tile (m2 = -inf); 1 for a row that has seen no
            // visible key yet (a caller mask can hide all of them)
            const float alpha = m_new == neg_inf() ? 1.f : exp2_fast(m2 - m_new);
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                o[db] *= alpha;
            l *= alpha;
            lr *= alpha;
            done[0] *= alpha;
            done[1] *= alpha;
            m2 = m_new;
            thr2 = m_new;
        }
    };

    // P = 2^(s c2 - m2) in fp32, summed into l (four independent chains); rounded to
    // T and packed in the MFMA B-operand order (chunk cc = 2kb + h holds registers
    // 8h .. 8h+7 of block kb); the rounded values summed into lr with v_dot2.  A row
    // with no visible key so far (m2 = -inf) gets p = 0.
    auto exp_sum_pack = [&](int j, f32x16* s, vec* pb) {
        const float mneg = (m2 == neg_inf()) ? 0.f : -m2;
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = exp2_fast(fmaf(s[cc >> 1][8 * (cc & 1) + e], c2, mneg));
                rs[e & 3] += p;
                pb[cc][e] = (T)p;
            }
        l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        float rr[2] = {0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const u32x4 w = __builtin_bit_cast(u32x4, pb[cc]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rr[e & 1] = M::dot_ones(w[e], rr[e & 1]);
        }
        lr += rr[0] + rr[1];
        if (j & 1)
            thr2 = m2 + (float)min(max(__builtin_amdgcn_frexp_expf(l) - kShift, 0), (int)kSlack);
        if ((j & (kSumBlock - 1)) == kSumBlock - 1) {
            done[0] += l;
            done[1] += lr;
            l = 0.f;
            lr = 0.f;
        }
        if (DROP) {
            // dropout on the P that multiplies V (l and lr keep the undropped P, the
            // keep scale is applied in the epilogue): chunk cc holds keys
            // 16cc + 4hh + 0..3 (e < 4) and 16cc + 8 + 4hh + 0..3 (e >= 4) of the tile
            const DropParams dp{prm.drop_key0, prm.drop_key1, prm.drop_t, prm.drop_keep_scale};
            uint32_t words[8];  // group 2cc + g: keys kbase + 16cc + 8g + 0..3
            drop_words_q8(dp, bh, my_q, kbeg + tile_of(j) * P::BC + 4 * hh, words);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                u32x4 w = __builtin_bit_cast(u32x4, pb[cc]);  // values 2i, 2i + 1 in word i
                uint32_t pw[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    drop_zero_pairs(words[2 * cc + g], pw + 2 * g, dp.t);
                pb[cc] = __builtin_bit_cast(vec, u32x4{pw[0], pw[1], pw[2], pw[3]});
            }
        }
    };

    // O^T += V^T P^T from the V buffer at vb_off
    auto pv = [&](const vec* pb, int vb_off) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                o[db] = M::mma(tr_operand<P::VSTR, vec>(sm + vb_off + tbase + 16 * cc * P::VSTR + 64 * db),
                               pb[cc], o[db]);
    };

    dma_barrier();  // publishes K_0, K_1, V_0 and V_1
    f32x16 sa[2], sb[2];
    float ma = 0.f, mb = 0.f;  // half-row maxima of the scores in sa / sb
    if (0 < ni_w) {
        scores(gbase + P::K0, sa);
        if (MASK)
            apply_mask_words(sa, mwd[0][0], mwd[0][1], hh);
        ma = tile_max(sa);
    }
    wg_barrier();  // every wave has read K_0
    if (2 < ni_g)
        stage_k(tile_of(2), P::K0);

    // One pipelined step of the group's local tile j (tile t = tile_of(j)): the
    // reference check for tile t (scores in s_cur, their half-row max in m_cur), then,
    // as one branch-free block, the S MFMAs of the group's next tile (K buffer kn, into
    // s_nxt) and their max, together with the softmax and P.V MFMAs of tile t (V^T
    // buffer vc); a wave's last tile is masked if it needs it and has no next tile.
    // Then the barrier publishes the K of local tile j + 2 and the V of local tile
    // j + 1 (DMA issued one step ago), and the next loads go out: V of local tile
    // j + 2 into vc, K of local tile j + 3 into kn.
    auto step = [&](int j, f32x16* s_cur, f32x16* s_nxt, float& m_cur, float& m_nxt, int kn,
                    int vc, auto SL) {
        constexpr int sl = decltype(SL)::value;  // mask-word slot of local tile j + 1
        if (j + 1 < ni_w) {
            update_max(m_cur);
            scores(gbase + kn, s_nxt);
            vec pb[4];
            exp_sum_pack(j, s_cur, pb);
            pv(pb, gbase + vc);
            if (MASK)
                apply_mask_words(s_nxt, mwd[sl][0], mwd[sl][1], hh);
            m_nxt = tile_max(s_nxt);
        } else if (j < ni_w) {
            if (needs_mask(tile_of(j))) {
                mask_tile(tile_of(j), s_cur);
                m_cur = tile_max(s_cur);
            }
            update_max(m_cur);
            vec pb[4];
            exp_sum_pack(j, s_cur, pb);
            pv(pb, gbase + vc);
        }
        dma_barrier();
        if (MASK && j + 2 < ni_w)
            load_mask(tile_of(j + 2), sl ^ 1);  // local tile j + 2 has the parity of j
        if (j + 2 < ni_g)
            stage_v(tile_of(j + 2), vc);
        if (j + 3 < ni_g)
            stage_k(tile_of(j + 3), kn);
    };
    for (int j = 0; j < ni; j += 2) {
        step(j, sa, sb, ma, mb, P::K1, P::V0, std::integral_constant<int, 1>{});
        if (j + 1 < ni)
            step(j + 1, sb, sa, mb, ma, P::K0, P::V1, std::integral_constant<int, 0>{});
    }

    // ---- key groups: the waves of groups 1 .. KG-1 hand their state to the group-0
    // wave of the same rows, which folds them in with the (+) operator of the
    // "Flash Attention" blog page on (m, d, o~): with M the largest reference,
    // o~ = sum_g 2^(m_g - M) o~_g and the same factors on both row sums (a group that
    // saw no key of the row has m_g = -inf and contributes nothing)
    float lsum = done[0] + l, lrsum = done[1] + lr;
    if (KG > 1) {
        constexpr int XW = 64 * (16 * P::DB + 4);  // floats per wave
        if (grp > 0) {
            float* const x = reinterpret_cast<float*>(smem + P::XOFF) +
                             ((grp - 1) * P::NQW + qw) * XW + lane * (16 * P::DB + 4);
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<f32x4*>(x + 16 * db + 4 * a) =
                        f32x4{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
            *reinterpret_cast<f32x4*>(x + 16 * P::DB) = f32x4{lsum, lrsum, m2, 0.f};
        }
        wg_barrier();
        if (grp > 0)
            return;  // no barrier follows
        const float* xg[KG - 1 > 0 ? KG - 1 : 1];
        float mg[KG - 1 > 0 ? KG - 1 : 1];
        float mx = m2;
#pragma unroll
        for (int g = 0; g < KG - 1; ++g) {
            xg[g] = reinterpret_cast<const float*>(smem + P::XOFF) + (g * P::NQW + qw) * XW +
                    lane * (16 * P::DB + 4);
            mg[g] = xg[g][16 * P::DB + 2];
            mx = fmaxf(mx, mg[g]);
        }
        // every row sees key 0 (tile 0 is group 0's), so m2 and mx are finite
        const float f0 = exp2_fast(m2 - mx);
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            o[db] *= f0;
        lsum *= f0;
        lrsum *= f0;
#pragma unroll
        for (int g = 0; g < KG - 1; ++g) {
            const float f = mg[g] == neg_inf() ? 0.f : exp2_fast(mg[g] - mx);
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 w = *reinterpret_cast<const f32x4*>(xg[g] + 16 * db + 4 * a);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[db][4 * a + e] = fmaf(f, w[e], o[db][4 * a + e]);
                }
            const f32x4 sums = *reinterpret_cast<const f32x4*>(xg[g] + 16 * P::DB);
            lsum = fmaf(f, sums[0], lsum);
            lrsum = fmaf(f, sums[1], lrsum);
        }
        m2 = mx;
    }

    if (!wave_active)
        return;  // no barrier follows

    // ---- epilogue: O = O~ / l (rounded to T, nearest-even), L = ln2 * (m2 + log2 l);
    // split: O~ / l and L in fp32 into the partial buffers, and for a row that saw
    // no key of its range the identity of the merge, L = -inf with O = 0
    const float lt = half_sum(lsum);
    const float lrt = half_sum(lrsum);
    // O goes through this wave's own LDS rows (the tile buffers are free after the
    // last barrier; the row sums lie past them), so that each store writes whole
    // rows rather than 8 or 16 bytes of 32 rows; fp32 partials 64 columns at a time
    char* const ost = smem + qw * 32 * P::OSTR;
    if (SPLIT) {
        const float inv = lrt > 0.f ? 1.0f / lrt : 0.f;
        float* const phead = prm.o_part + ((size_t)split * prm.bh_count + bh) * Nq * D;
#pragma unroll
        for (int half = 0; half < D / 64; ++half) {
#pragma unroll
            for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = o[db][4 * a + e] * inv;
                    *reinterpret_cast<f32x4*>(ost + ql * P::OSTR + 4 * (32 * (db - 2 * half) + 8 * a + 4 * hh)) = w;
                }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + (lane >> 4);
                const int ch = lane & 15;
                const f32x4 piece = *reinterpret_cast<const f32x4*>(ost + r * P::OSTR + 16 * ch);
                if (qw0 + r < Nq)
                    *reinterpret_cast<f32x4*>(phead + (size_t)(qw0 + r) * D + 64 * half + 4 * ch) = piece;
            }
        }
        if (hh == 0 && my_q < Nq)
            prm.lse_part[((size_t)split * prm.bh_count + bh) * Nq + my_q] =
                lt > 0.f ? (m2 + log2_fast(lt)) * kLn2 : neg_inf();
    } else {
        // a row that saw no visible key (only with a caller mask): O = 0, L = -inf
        const float inv = (MASK && !(lrt > 0.f)) ? 0.f : (DROP ? prm.drop_keep_scale : 1.0f) / lrt;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (T)(o[db][4 * a + e] * inv);
                *reinterpret_cast<T4*>(ost + ql * P::OSTR + 2 * (32 * db + 8 * a + 4 * hh)) = w;
            }
        constexpr int LPR = 2 * D / 16;  // lanes per row of T, 16 bytes each
        constexpr int RPI = 64 / LPR;    // rows per store
        T* const ohead = prm.o + (size_t)bh * Nq * D;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = RPI * i + lane / LPR;
            const int ch = lane % LPR;
            const u32x4 piece = *reinterpret_cast<const u32x4*>(ost + r * P::OSTR + 16 * ch);
            if (qw0 + r < Nq)
                *reinterpret_cast<u32x4*>(ohead + (size_t)(qw0 + r) * D + 8 * ch) = piece;
        }
        if (hh == 0 && my_q < Nq)
            prm.lse[(size_t)bh * Nq + my_q] =
                (MASK && !(lt > 0.f)) ? neg_inf() : (m2 + log2_fast(lt)) * kLn2;
    }
}

}  // namespace fa
