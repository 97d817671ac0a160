// fa_fwd_pp.hpp — fused attention forward for bf16 / fp16 inputs and d = 128 on
// gfx950, with the two waves of every SIMD in alternating phases.
//
// The arithmetic is that of fa_fwd_mfma16.hpp (the course page "05_flash_attention.py",
// flash_attention_forward: per query tile m = -inf, l = 0, O~ = 0; per key/value tile
// S = Q K_j^T scale, m_new = max(m, rowmax S), P = exp(S - m_new), l = alpha l +
// rowsum P, O~ = alpha O~ + P V_j; O = O~ / l and L = m + log l at the end), with the
// same transposed 32x32x16 MFMA formulation, reference-max rule and two row sums.
// What differs is the schedule.
//
// A workgroup is 8 waves (256 query rows) and fills a CU; waves w and w + 4 share a
// SIMD.  Waves 0-3 form group 0, waves 4-7 group 1, and the two groups run in
// opposite phases separated by workgroup barriers:
//   * an MFMA phase of tile j, at raised wave priority: S_{j+1} = K_{j+1} Q^T (16
//     MFMAs) and O~ += V_j^T P_j^T (16 MFMAs), operands read from LDS, then the mask
//     and the running max of tile j+1 (VALU work behind the last MFMAs, in the time
//     the phase would otherwise wait at its barrier);
//   * a softmax phase of tile u: P_u = 2^(S_u c - m) rounded to T, the two row
//     sums, plus the wave's share of the staging: its DMA blocks of K_{u+2} and of
//     V_{u+1}.  (Tile 0's mask and max run in the first softmax phase, and with
//     dropout every tile's, as before the move.)
// While one wave of a SIMD issues its 32 MFMAs back to back, the other wave's
// softmax instructions take the issue slots the matrix core leaves free, instead of
// both waves contending for the same slots in the same phase:
//     phase 2j:    group 0 MFMA(j),     group 1 softmax(j)
//     phase 2j+1:  group 0 softmax(j+1), group 1 MFMA(j)
// Query rows: the two waves of SIMD s own the tile's 32-row blocks s (wave s, group 0)
// and 7 - s (wave s + 4, group 1).  Under a causal mask block b's last row sees key
// tile q0 / 64 + b / 2 (b / 2 rounded down) last, so the blocks' tile counts run from
// nkt - 3 (blocks 0, 1) to nkt (blocks 6, 7); pairing the short and long blocks leaves one
// active wave per SIMD in the workgroup's last two tile steps, whose phases then run
// without the other wave's interference, instead of leaving whole SIMDs idle while the
// SIMD that holds blocks 6 and 7 runs both at the full phase length.
//
// Staging, K and V both by DMA (buffer_load ... lds), three buffers each.  K rows
// are padded to 272 bytes (as in fa_fwd_mfma16.hpp): the 16 rows of one
// ds_read_b128 pass fall in distinct banks.  V stays row-major, rows padded to 320
// bytes, and the A operand of O^T = V^T P^T (32 dims x 16 keys, a lane holding 8
// keys of one dim) comes from two ds_read_b64_tr_b16, gfx950's transposing LDS
// read: each group of 16 lanes reads 4 rows x 16 dims and receives them transposed,
// lane j dim j with the 4 rows in order; with 320-byte rows the 4 rows of a
// half-wave's read sit 16 banks apart.  The keys land in the k-slots that the
// rounded P occupies (slot 8h + 4r + e of chunk cc holds key 16cc + 8r + 4h + e, as
// the 32x32 accumulator layout gives it).  Group 0 issues its blocks of K_t in the
// softmax phase of tile t-2 (phase 2t-5) and of V_t in that of tile t-1 (phase
// 2t-3); group 1 one tile earlier, K_t in phase 2t-6 and V_t in phase 2t-4.  A group
// waits for its loads at the end of its following MFMA phase, so all of K_t has
// landed by the end of phase 2t-4 and all of V_t by the end of phase 2t-2.  Each wave
// reads the operands of the first MFMA pairs of its MFMA phase at the start of the
// softmax phase before it (group 0 reads K_t first in phase 2t-3, V_t in phase
// 2t-1), and no buffer is rewritten before its last reader's phase has ended (K_t
// and V_t go where K_{t-3} and V_{t-3} were, last read in phases 2t-7 and 2t-5).
//
// Q and O move as whole rows: the prologue stages the workgroup's 256 Q rows by DMA
// into buffers not yet in use and each wave reads its fragments from there; the
// epilogue writes O (or the fp32 partials) through each wave's own LDS rows.  The
// workgroup's (head, query tile) comes from work_item (fa_common.hpp).
//
// With key splits a workgroup stages one range of whole key tiles and writes fp32
// partial states, as fa_fwd_mfma16.hpp does; with dropout the softmax phase zeroes
// the dropped entries of the rounded P (the Philox words of fa_philox.hpp); with a
// caller mask (the blog page "Flash Attention", Algorithm 2: S_masked = mask(S)) the
// hidden scores are set to -inf from the mask words, loaded one tile ahead, just
// before the running max is taken (at the end of the MFMA phase before the tile's
// softmax phase; for tile 0 at the start of the first softmax phase), and a row that
// sees no key ends with O = 0 and L = -inf.
#pragma once

#include <type_traits>

#include "fa_philox.hpp"
#include "fa_tiles.hpp"

namespace fa {

struct TilePP {
    static constexpr int D = 128;
    static constexpr int NW = 8;              // waves per workgroup
    static constexpr int BR = 256;            // query rows per workgroup
    static constexpr int BC = 64;             // keys per K/V tile
    static constexpr int NT = 512;            // threads per workgroup
    static constexpr int KSTR = 2 * D + 16;   // K row stride in LDS
    static constexpr int VSTR = 2 * D + 64;   // V row stride in LDS
    static constexpr int KT = BC * KSTR;      // bytes of one K tile in LDS
    static constexpr int VT = BC * VSTR;      // bytes of one V tile in LDS
    static constexpr int KNB = KT / 1024;     // 1-KB DMA blocks per K tile
    static constexpr int KPW = (KNB + NW - 1) / NW;
    static constexpr int VNB = VT / 1024;     // 1-KB DMA blocks per V tile
    static constexpr int VPW = (VNB + NW - 1) / NW;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int NKB = 3;             // K buffers
    static constexpr int NVB = 3;             // V buffers
    static constexpr int VOFF = NKB * KT;     // first V buffer
    static constexpr int LDS = NKB * KT + NVB * VT;
    static constexpr int OSTR = 2 * D + 16;   // bytes per row of a wave's O in LDS (epilogue)
    static_assert(NW * 32 * OSTR <= LDS, "the epilogue's O rows must fit the K and V^T buffers");
    static_assert(KT + BR * KSTR <= LDS, "the prologue's Q rows must fit past K buffer 0");
    static_assert(KT % 1024 == 0 && VT % 1024 == 0, "tiles must be whole DMA blocks");
};

// s_waitcnt immediates (gfx9 encoding): LDS only, and all memory
constexpr int kWaitLds = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitAll = 0x0070;  // vmcnt(0) lgkmcnt(0)

template <typename T, bool CAUSAL, bool SPLIT, bool DROP = false, bool MASK = false>
__global__ __launch_bounds__(TilePP::NT) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_pp_kernel(const FwdParams<T> prm)
{
    using P = TilePP;
    using M = Mfma16<T>;
    using vec = typename M::vec;
    constexpr int D = P::D;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const char* const sm = smem;
    const int Nq = prm.Nq, Nk = prm.Nk, n_qtiles = prm.n_qtiles;
    const float c2 = prm.c2;

    // ---- (batch*head, key split, query tile) of this workgroup: the query tiles of
    // one (head, split) share an XCD; causal: the longest rows (most key tiles) first
    const WorkItem wi = work_item((int)blockIdx.x, (int)gridDim.x, n_qtiles, CAUSAL && !SPLIT);
    const int rest = wi.head;
    const int qt = CAUSAL ? n_qtiles - 1 - wi.rank : wi.rank;
    const int split = SPLIT ? rest % prm.n_splits : 0;
    const int bh = SPLIT ? rest / prm.n_splits : rest;
    const int q0 = qt * P::BR;

    const int tid = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // ping-pong group (wave-uniform)
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int qw0 = q0 + 32 * (grp == 0 ? (wave & 3) : 7 - (wave & 3));
    const int my_q = qw0 + ql;

    // ---- key range: keys [kbeg, kbeg + Nks) of the head (all of them unless split);
    // key tiles and positions below are relative to kbeg, so a query's causal limit is
    // its index minus kbeg.  kbeg is a multiple of 64, so a wave's 32 rows either all
    // see key kbeg or see no key of the range.
    const int kbeg = SPLIT ? split * prm.split_tiles * P::BC : 0;
    const int Nks = SPLIT ? min(Nk - kbeg, prm.split_tiles * P::BC) : Nk;
    const T* Qh = prm.q + (size_t)bh * Nq * D;
    const T* Kh = prm.k + ((size_t)bh * Nk + kbeg) * D;
    const T* Vh = prm.v + ((size_t)bh * Nk + kbeg) * D;

    // ---- key tiles: the workgroup stages nkt, this wave computes n_w
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

    // ---- staging: this wave's DMA blocks of K and V tiles.  The 1-KB blocks of a tile
    // are dealt round-robin starting with group 1 (slot = (wave + 4) % 8), so the blocks
    // past the first 16 (K's 17th, V's 17th to 20th) fall to group 1: it issues 21 of a
    // tile's 37 blocks and group 0 16, and less of the DMA data lands during the phase
    // in which group 1's softmax (the longer of the two softmax phases) runs.  Measured
    // +0.5-1 % over the other way round on one box and within +-0.2 % on another;
    // moving all of the staging to group 1 was mixed (-1.3 to +0.4 %).
    const int slot = (wave + 4) & (P::NW - 1);
    int ksrc[P::KPW], vsrc[P::VPW];
#pragma unroll
    for (int i = 0; i < P::KPW; ++i)
        ksrc[i] = dma_src<D>(slot + P::NW * i, lane, P::KSTR);
#pragma unroll
    for (int i = 0; i < P::VPW; ++i)
        vsrc[i] = dma_src<D>(slot + P::NW * i, lane, P::VSTR);
    auto stage_k = [&](int t, int lds_off) {
        stage_tile<D, P::KNB, P::KPW, P::NW>(Kh, t, Nks, smem + lds_off, slot, ksrc);
    };
    auto stage_v = [&](int t, int lds_off) {
        stage_tile<D, P::VNB, P::VPW, P::NW>(Vh, t, Nks, smem + lds_off, slot, vsrc);
    };

    // ---- caller mask: this lane's row of the head's mask slice, the words of one tile
    // loaded a tile ahead (slot = tile % 2); the workgroup's rows bound the resource
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

    const int kbase = ql * P::KSTR + hh * 16;
    // transposing V reads: lane (h = lane / 32, g = (lane / 16) % 2, j = lane % 16)
    // addresses row 4h + j / 4 (plus 8r + 16cc) at dims 16g + 4 (j % 4) .. +3 (plus 32db)
    const int vbase = (4 * hh + ((lane >> 2) & 3)) * P::VSTR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    // ---- Q fragment (B operand of S^T = K Q^T): lane supplies Q[my_q][16c + 8hh .. +8],
    // read in the prologue from the workgroup's Q rows staged in LDS (rows past Nq are 0)
    vec qf[P::DC];

    // ---- running state
    f32x16 o[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        o[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    f32x16 s[2];  // S^T of the tile whose softmax is next
    vec pb[4];    // P of the tile whose P.V is next, rounded, B-operand order
    float m2 = neg_inf();
    // Row sums of this half: ls0, ls1 of the fp32 P (for L) and lrs0, lrs1 of the rounded P
    // (for the normalisation of O), independent chains that run across the tiles of
    // a block of kSumBlock key tiles and are folded into l_done / lr_done when the
    // block ends.  A sequential fp32 sum over T tiles can drift by up to about
    // T 2^-24 of its value (when the tile sums are alike); blocks bound the drift by
    // about (kSumBlock + T / kSumBlock) 2^-24.
    float ls0 = 0.f, ls1 = 0.f, lrs0 = 0.f, lrs1 = 0.f;
    float l_done = 0.f, lr_done = 0.f;
    bool rescale = false;  // a rescale of O~ by alpha is pending (see update_max)
    float alpha = 1.f;

    // S^T of one tile from the K buffer at kb_off
    auto scores_only = [&](int kb_off) {
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
    // The operands of the first NPRE MFMA pairs (pair i: S^T MFMA i, P.V MFMA i) of an
    // MFMA phase, read at the start of the softmax phase before it, so that the MFMA
    // phase starts on operands already in registers (their tiles have landed by then:
    // see the staging schedule above).
    constexpr int NPRE = 2;  // one, three or four pairs time 0.5-1 % slower
    vec pre_k[NPRE], pre_v[NPRE];
    auto pre_read = [&](int kb_off, int vb_off) {
#pragma unroll
        for (int i = 0; i < NPRE; ++i) {
            const int c = i >> 1, kb = i & 1, cc = i >> 2, db = i & 3;
            pre_k[i] = *reinterpret_cast<const vec*>(sm + kb_off + kbase + 32 * c + kb * 32 * P::KSTR);
            pre_v[i] = tr_operand<P::VSTR, vec>(sm + vb_off + vbase + 16 * cc * P::VSTR + 64 * db);
        }
    };
    // both, interleaved: S^T of tile j+1 and P.V of tile j; the operand reads run
    // four MFMAs ahead (a fixed DS-read / MFMA order keeps the operands in flight,
    // and their registers, bounded)
    auto scores_pv = [&](int kb_off, int vb_off) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            s[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = i >> 1, kb = i & 1;
            const vec a = i < NPRE ? pre_k[i]
                                   : *reinterpret_cast<const vec*>(sm + kb_off + kbase + 32 * c + kb * 32 * P::KSTR);
            s[kb] = M::mma(a, qf[c], s[kb]);
            const int cc = i >> 2, db = i & 3;
            const vec b = i < NPRE ? pre_v[i]
                                   : tr_operand<P::VSTR, vec>(sm + vb_off + vbase + 16 * cc * P::VSTR + 64 * db);
            o[db] = M::mma(b, pb[cc], o[db]);
        }
        // the preloaded pairs first, each followed by the reads of the pair NPRE ahead
        // (3 each: one K, two V), then per MFMA pair the reads of the pair NPRE ahead,
        // so that the operands stay 2 NPRE MFMAs ahead
#pragma unroll
        for (int i = 0; i < NPRE; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
#pragma unroll
        for (int i = 0; i < 16 - 2 * NPRE; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NPRE, 0);
    };

    // Mask of tile j (keys past the end, or after the query): only a wave's last
    // tile can need it (its first query is a multiple of 32, tiles are 64 keys).
    auto needs_mask = [&](int j) {
        const int key0 = j * P::BC;
        return (key0 + P::BC > Nks) || (CAUSAL && key0 + P::BC - 1 > qw0 - kbeg);
    };
    auto mask_tile = [&](int j) {
        const int key0 = j * P::BC;
        const int last = CAUSAL ? min(Nks - 1, my_q - kbeg) : Nks - 1;
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

    // Running max with a reference that moves only when it matters (as in
    // fa_fwd_mfma16.hpp): the reference m2 moves to the rows' maxima, with the rescale
    // of O~ and the row sums by 2^(m2 - m_new), when some row's tile max exceeds
    // m2 + g, g = clamp(e - kShift, 0, kSlack), where e is the binary exponent of a
    // lower bound of the row's running sum l (l >= 2^(e-1)): this half's part of it,
    // from an earlier tile (l only grows between moves).  A key that does not move the
    // reference has P <= 2^g <= l / 4, so it weighs at most 1/5 of its row, and
    // P <= 2^kSlack.  A key that does gets P = 1 exactly, as in the pages' recurrence
    // (which moves on every new maximum): the weight of a row's dominant key is not
    // rounded, and while l is small (peaked rows, a row's first tiles) every new
    // maximum moves the reference.  O is divided by the sum of the same rounded P that
    // entered the P.V MFMAs, L uses the fp32 sum.  The rescale of O~ is applied by the
    // next MFMA phase (O~ is touched by MFMA phases only): `rescale` marks it pending,
    // alpha holds the factor.  What the per-tile work needs of m2 is kept ready:
    // mneg = -m2 (0 while m2 = -inf, so that a row with no visible key gets p = 0) and
    // the raw-score threshold thr = (m2 + g) / c2 of the move test (c2 > 0): g = 0
    // after a move, recomputed every second tile.
    constexpr float kSlack = 8.0f;
    constexpr int kShift = 3;
    const float inv_c2 = 1.0f / c2;
    float mneg = 0.f, thr = neg_inf();
    auto update_max = [&]() {
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[kb][r]);
        if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
            const float mh = mx * c2;  // c2 > 0: max commutes with the scale
            const float m_new = fmaxf(m2, half_max(mh));
            // 0 on a row's first visible tile (m2 = -inf); 1 for a row that has seen no
            // visible key yet (a caller mask can hide all of them)
            alpha = m_new == neg_inf() ? 1.f : exp2_fast(m2 - m_new);
            rescale = true;
            ls0 *= alpha;
            ls1 *= alpha;
            lrs0 *= alpha;
            lrs1 *= alpha;
            l_done *= alpha;
            lr_done *= alpha;
            m2 = m_new;
            mneg = (m_new == neg_inf()) ? 0.f : -m_new;
            thr = m_new * inv_c2;
        }
    };
    // threshold of the move test from the current sums (m2 = -inf keeps it at -inf)
    auto update_thr = [&]() {
        const int e = __builtin_amdgcn_frexp_expf(l_done + (ls0 + ls1));
        thr = (m2 + (float)min(max(e - kShift, 0), (int)kSlack)) * inv_c2;
    };
    // P = 2^(s c2 - m2) in fp32, summed into ls; rounded to T in the MFMA B-operand
    // order (chunk cc = 2kb + h holds registers 8h .. 8h+7 of block kb); the rounded
    // values summed into lrs with v_dot2.
    auto exp_sum_pack = [&]() {
        float rs[2] = {ls0, ls1};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = exp2_fast(fmaf(s[cc >> 1][8 * (cc & 1) + e], c2, mneg));
                rs[e & 1] += p;
                pb[cc][e] = (T)p;
            }
        ls0 = rs[0];
        ls1 = rs[1];
        float rr[2] = {lrs0, lrs1};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const u32x4 w = __builtin_bit_cast(u32x4, pb[cc]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rr[e & 1] = M::dot_ones(w[e], rr[e & 1]);
        }
        lrs0 = rr[0];
        lrs1 = rr[1];
    };
    // softmax phase of tile u; forced inline, since with dropout the compiler would
    // otherwise emit it as a function and keep the captured state in scratch memory
    auto softmax = [&](int u, auto UPD, auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value;
        if (u < n_w) {
            if (u == 0 || DROP) {
                if (needs_mask(u))
                    mask_tile(u);
                if (MASK)
                    apply_mask_words(s, mwd[r & 1][0], mwd[r & 1][1], hh);
                update_max();
            }
            exp_sum_pack();
            if (decltype(UPD)::value)
                update_thr();
            if (DROP) {
                // dropout on the P that multiplies V (the row sums keep the undropped P,
                // the keep scale is applied in the epilogue): chunk cc holds keys
                // 16cc + 4hh + 0..3 (e < 4) and 16cc + 8 + 4hh + 0..3 (e >= 4) of the tile
                const DropParams dp{prm.drop_key0, prm.drop_key1, prm.drop_t, prm.drop_keep_scale};
                uint32_t words[8];  // group 2cc + g: keys 16cc + 8g + 4hh + 0..3 of the tile
                drop_words_q8(dp, bh, my_q, kbeg + u * P::BC + 4 * hh, words);
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
            if ((u & (kSumBlock - 1)) == kSumBlock - 1) {
                l_done += ls0 + ls1;
                lr_done += lrs0 + lrs1;
                ls0 = ls1 = 0.f;
                lrs0 = lrs1 = 0.f;
            }
        }
    };
    // MFMA phase of tile j (j = R mod 6): S^T of tile j+1 and P.V of tile j (K buffer
    // of tile j+1, V buffer of tile j).  On a wave's last tile the
    // S^T MFMAs read a K buffer that holds no tile of this wave (stale but allocated
    // LDS) and their result is never used: one code path keeps O~ in the same
    // registers throughout the loop.  The phase runs at raised wave priority, so the
    // SIMD's arbiter issues this wave's MFMAs ahead of the other group's VALU work.
    auto mfma = [&](int j, auto R) {
        constexpr int r = decltype(R)::value;
        __builtin_amdgcn_s_setprio(3);
        if (rescale) {
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                o[db] *= alpha;
            rescale = false;
        }
        if (j < n_w)
            scores_pv(((r + 1) % P::NKB) * P::KT, P::VOFF + (r % P::NVB) * P::VT);
        // the mask and running max of tile j+1, here rather than at the start of its
        // softmax phase: the same state updates in the same order (tile j's sums and
        // threshold are complete, the rescale of O~ still waits for the next MFMA
        // phase), but issued while the last MFMAs run, which shortens the softmax
        // phase, the longer of the two (+0.4 to +2.2 % on three shapes; also moving
        // the exp of the tile's first chunk here was 1-2 % slower).  Not with
        // dropout, whose softmax phase keeps its own order.
        if (!DROP && j + 1 < n_w) {
            if (needs_mask(j + 1))
                mask_tile(j + 1);
            if (MASK)
                apply_mask_words(s, mwd[(r + 1) & 1][0], mwd[(r + 1) & 1][1], hh);
            update_max();
        }
    };
    // staging in the softmax phase of tile u (u = R mod 6): the operands of the first
    // MFMA pairs of MFMA(u) (ahead of the DMA: the compiler makes every transposing
    // LDS read wait for all of the wave's DMA in flight), then this wave's DMA blocks
    // of K_{u+2} and V_{u+1} (group 0) or K_{u+3} and V_{u+2} (group 1); the phase runs
    // at normal priority
    auto stage = [&](int u, auto R) {
        constexpr int r = decltype(R)::value;
        __builtin_amdgcn_s_setprio(0);
        if (u < n_w)
            pre_read(((r + 1) % P::NKB) * P::KT, P::VOFF + (r % P::NVB) * P::VT);
        if (MASK && u + 1 < n_w)
            load_mask(u + 1, (r + 1) & 1);
        if (grp == 0) {
            if (u + 2 < nkt)
                stage_k(u + 2, ((r + 2) % P::NKB) * P::KT);
            if (u + 1 < nkt)
                stage_v(u + 1, P::VOFF + ((r + 1) % P::NVB) * P::VT);
        } else {
            if (u + 3 < nkt)
                stage_k(u + 3, (r % P::NKB) * P::KT);
            if (u + 2 < nkt)
                stage_v(u + 2, P::VOFF + ((r + 2) % P::NVB) * P::VT);
        }
    };    // end of a phase: this wave's LDS traffic (and, after an MFMA phase, its loads)
    // complete, then the workgroup barrier
    auto barrier = [&](bool loads) {
        __asm__ volatile("" ::: "memory");
        if (loads || kFullBarrier)
            __builtin_amdgcn_s_waitcnt(kWaitAll);
        else
            __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    // ---- prologue: K_0 and the workgroup's 256 Q rows by DMA (Q into the buffers past
    // K buffer 0, free until K_1 and V_0 arrive; whole rows per DMA block, where
    // loading the fragments straight from memory would touch 32 rows per load).  Then
    // every wave reads its Q fragments, and a barrier frees the area for K_1 and V_0.
    if (0 < nkt)
        stage_k(0, 0);
#pragma unroll
    for (int t = 0; t < P::BR / P::BC; ++t)
        stage_tile<D, P::KNB, P::KPW, P::NW>(Qh, q0 / P::BC + t, Nq, smem + P::KT * (1 + t), slot, ksrc);
    if (MASK && 0 < n_w)
        load_mask(0, 0);
    barrier(true);
    {
        const char* const qrow = sm + P::KT + (qw0 - q0 + ql) * P::KSTR + hh * 16;
#pragma unroll
        for (int c = 0; c < P::DC; ++c)
            qf[c] = *reinterpret_cast<const vec*>(qrow + 32 * c);
    }
    barrier(false);
    if (0 < nkt)
        stage_v(0, P::VOFF);
    if (1 < nkt && grp == 0)
        stage_k(1, P::KT);

    // ---- phases: group 0 runs MFMA(j) in phase 2j and softmax(u) in phase 2u - 1,
    // group 1 softmax(u) in phase 2u and MFMA(j) in phase 2j + 1.  Both groups run
    // the same code, one MFMA and one softmax phase per iteration; group 1 enters
    // one phase later (it issues its K_1, K_2 and V_1 blocks in phase -2, while group
    // 0 computes S_0) and group 0 closes with one barrier more, so both pass the same
    // barriers.  V_0 and K_1 land before the first barrier that waits for loads.
    if (grp == 1) {
        if (1 < nkt)
            stage_k(1, P::KT);
        if (2 < nkt)
            stage_k(2, 2 * P::KT);
        if (1 < nkt)
            stage_v(1, P::VOFF + P::VT);
        barrier(true);
    }
    if (0 < n_w)
        scores_only(0);
    barrier(true);
    stage(0, std::integral_constant<int, 0>{});
    softmax(0, std::false_type{}, std::integral_constant<int, 0>{});
    barrier(false);
    // unrolled by 6 = lcm(3 buffers, the tile parity of the mask words and of the
    // threshold update), so that every buffer offset and register slot is a constant
    auto iter = [&](int j, auto R) {  // j = R (mod 6)
        constexpr int r = decltype(R)::value;
        mfma(j, R);
        barrier(true);
        stage(j + 1, std::integral_constant<int, (r + 1) % 6>{});
        softmax(j + 1, std::integral_constant<bool, (r & 1) == 0>{},  // odd tiles
                std::integral_constant<int, (r + 1) % 6>{});
        barrier(false);
    };
    for (int j = 0; j < nkt; j += 6) {
        iter(j, std::integral_constant<int, 0>{});
        if (j + 1 < nkt)
            iter(j + 1, std::integral_constant<int, 1>{});
        if (j + 2 < nkt)
            iter(j + 2, std::integral_constant<int, 2>{});
        if (j + 3 < nkt)
            iter(j + 3, std::integral_constant<int, 3>{});
        if (j + 4 < nkt)
            iter(j + 4, std::integral_constant<int, 4>{});
        if (j + 5 < nkt)
            iter(j + 5, std::integral_constant<int, 5>{});
    }
    if (grp == 0)
        barrier(false);

    if (!wave_active)
        return;  // no barrier follows
    // ---- epilogue: O = O~ / lr (times the keep scale with dropout, rounded to T),
    // L = ln2 (m2 + log2 l); split: O~ / lr
    // and L in fp32 into the partial buffers, and for a row that saw no key of its
    // range the identity of the merge, L = -inf with O = 0
    const float lsum = l_done + (ls0 + ls1);
    const float lrsum = lr_done + (lrs0 + lrs1);
    const float lt = half_sum(lsum);
    const float lrt = half_sum(lrsum);
    if (SPLIT) {
        // fp32 partial O through this wave's LDS rows as below, in two halves of 64
        // columns (256 bytes a row, like a row of T)
        const float inv = lrt > 0.f ? 1.0f / lrt : 0.f;
        char* const ost = smem + wave * 32 * P::OSTR;
        float* const phead = prm.o_part + ((size_t)split * prm.bh_count + bh) * Nq * D;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
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
        return;
    }
    // O rounded to T goes through this wave's own LDS rows (the K and V^T buffers are
    // free after the last barrier), so that each store writes four whole rows of O
    // rather than 16-byte pieces of 32 rows
    // a row that saw no visible key (only with a caller mask): O = 0, L = -inf
    const float inv = (MASK && !(lrt > 0.f)) ? 0.f : (DROP ? prm.drop_keep_scale : 1.0f) / lrt;
    char* const ost = smem + wave * 32 * P::OSTR;
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
    T* const ohead = prm.o + (size_t)bh * Nq * D;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int ch = lane & 15;
        const u32x4 piece = *reinterpret_cast<const u32x4*>(ost + r * P::OSTR + 16 * ch);
        if (qw0 + r < Nq)
            *reinterpret_cast<u32x4*>(ohead + (size_t)(qw0 + r) * D + 8 * ch) = piece;
    }
    if (hh == 0 && my_q < Nq)
        prm.lse[(size_t)bh * Nq + my_q] =
            (MASK && !(lt > 0.f)) ? neg_inf() : (m2 + log2_fast(lt)) * kLn2;
}

}  // namespace fa
