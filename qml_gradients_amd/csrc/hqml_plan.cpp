// Host scheduler for the fused training step (no HIP calls).
//
// Forward gate fusion (hugo-pages summary, section 1.4 item 1): each fused pass
// reads a state once, applies a block of gates on chip and writes the block's
// output once.  A tile view keeps 13 of the n qubits on chip; rotations of one
// layer commute across qubits, so each layer's real rotations are split into one
// group per view, and consecutive layers are interleaved so that a pass applies
// [group of layer l, merged diagonal D_l, the same group of layer l+1].  With two
// views (14 <= n <= 20) that is one pass per layer; with V views, V-1 passes.
#include "hqml_plan.hpp"

#include <algorithm>
#include <cstdio>
#include <cstring>

namespace hqml {

namespace {

constexpr int kLowQubits = 4;   // positions 0..3 always hold qubits 0..3 (128-byte runs)

// Register positions of the two layouts (see hqml_internal.hpp): L1 rotates positions
// 4..8, L2 positions 0, 1, 9, 10, 11.
constexpr uint32_t kL1Regs = 0x1F0u;
constexpr uint32_t kL2Regs = 0xE03u;

// Whether qubits a and b are neighbours in the CZ chain.
bool adjacent(int a, int b) { return a >= 0 && b >= 0 && (a - b == 1 || b - a == 1); }

// Check a view's placement: (a) no qubit at a register position of a layout is a chain
// neighbour of a rotated qubit at a register position of the same layout (so the sign of
// Z_{q-1} Z_{q+1} is constant over a thread's registers wherever the statistics of a
// rotated qubit q are taken); (b) no qubit at L2 positions 0, 1 neighbours one at 9..11
// (the diagonal's per-thread factor tables handle CZ signs within those two sets only).
bool view_ok(const int *perm, uint32_t group)
{
    for (uint32_t regs : {kL1Regs, kL2Regs})
        for (int a = 0; a < kTileBits; ++a) {
            if (!((regs >> a) & 1u) || !((group >> a) & 1u)) continue;
            for (int b = 0; b < kTileBits; ++b)
                if (b != a && ((regs >> b) & 1u) && adjacent(perm[a], perm[b])) return false;
        }
    for (int a : {0, 1})
        for (int b : {9, 10, 11})
            if (adjacent(perm[a], perm[b])) return false;
    return true;
}

// Views.  Qubit q is rotated by view q mod V, so no two chain neighbours share a view:
// the rotations of a pass never touch the neighbours of the qubits it rotates, and the
// backward pass can take both of its layers' statistics from one point (the merged
// statistics of the adjoint kernel).  V = max(2, ceil((n - 4) / 8)) views keep at most
// 8 high qubits (>= 4) and 2 low qubits per view on the 10 rotatable positions.  A
// view's rotated low qubits sit at positions 0, 1 (the other low qubits at 2, 3 or as
// fillers of 0, 1), its rotated high qubits at 4..8 (L1 registers) and 9..11 (L2
// registers), and the remaining register positions, position 12 and the tile bits take
// the other qubits, subject to view_ok.
bool build_views(int n, Plan &p, std::string *err)
{
    const int nhigh = n - kLowQubits;
    const int V = std::max(2, (nhigh + 7) / 8);
    p.V = V;
    p.T = 1 << (n - kTileBits);
    p.views.assign(V, ViewDev{});
    for (int v = 0; v < V; ++v) {
        std::vector<int> rlow, rhigh, olow, ohigh;
        for (int q = 0; q < n; ++q) {
            const bool mine = q % V == v;
            if (q < kLowQubits) (mine ? rlow : olow).push_back(q);
            else (mine ? rhigh : ohigh).push_back(q);
        }
        if (rlow.size() > 2 || rhigh.size() > 8) {
            if (err) *err = "a view has more rotated qubits than rotatable positions";
            return false;
        }
        std::sort(ohigh.rbegin(), ohigh.rend());   // fillers: highest first
        const int kh = (int)rhigh.size();
        bool placed = false;
        int perm[kTileBits];
        uint32_t group = 0;
        // Try every choice of the rotated high qubits that go to L2 (highest first), and
        // every low filler order, until the placement passes view_ok.
        const int nl2_min = std::max(0, kh - 5), nl2_max = std::min(3, kh);
        for (int nl2 = nl2_min; nl2 <= nl2_max && !placed; ++nl2) {
            std::vector<int> pick(kh, 0);
            std::fill(pick.end() - nl2, pick.end(), 1);
            do {
                std::vector<int> lo2 = olow;
                std::sort(lo2.begin(), lo2.end());
                do {
                    for (int i = 0; i < kTileBits; ++i) perm[i] = -1;
                    group = 0;
                    std::vector<int> low = rlow;
                    for (int q : lo2) low.push_back(q);
                    for (int i = 0; i < kLowQubits; ++i) perm[i] = low[i];
                    for (size_t i = 0; i < rlow.size(); ++i) group |= 1u << i;
                    int p1 = 4, p2 = 9;
                    for (int k = 0; k < kh; ++k) {
                        const int pos = pick[k] ? p2++ : p1++;
                        perm[pos] = rhigh[k];
                        group |= 1u << pos;
                    }
                    std::vector<int> cand = ohigh;
                    bool ok = true;
                    for (int pos = 4; pos < kTileBits && ok; ++pos) {
                        if (perm[pos] >= 0) continue;
                        const uint32_t regs = ((kL1Regs >> pos) & 1u) ? kL1Regs : ((kL2Regs >> pos) & 1u) ? kL2Regs : 0u;
                        ok = false;
                        for (size_t ci = 0; ci < cand.size(); ++ci) {
                            bool clash = false;
                            for (int b = 0; b < kTileBits && regs; ++b)
                                if (((regs >> b) & 1u) && ((group >> b) & 1u) && adjacent(cand[ci], perm[b])) clash = true;
                            if (!clash) {
                                perm[pos] = cand[ci];
                                cand.erase(cand.begin() + (long)ci);
                                ok = true;
                                break;
                            }
                        }
                    }
                    if (ok && view_ok(perm, group)) placed = true;
                } while (!placed && std::next_permutation(lo2.begin(), lo2.end()));
            } while (!placed && std::next_permutation(pick.begin(), pick.end()));
        }
        if (!placed) {
            if (err) *err = "no tile view keeps the chain neighbours of its rotated qubits off its register positions";
            return false;
        }
        ViewDev &d = p.views[v];
        std::memset(&d, 0, sizeof(d));
        for (int i = 0; i < 32; ++i) d.inv[i] = -1;
        for (int i = 0; i < kTileBits; ++i) {
            d.perm[i] = perm[i];
            d.inv[perm[i]] = i;
        }
        d.group_mask = (int32_t)group;
        int nt = 0;
        for (int q = 0; q < n; ++q)
            if (d.inv[q] < 0) d.tile_q[nt++] = q;
        d.n_tile = nt;
        if (nt != n - kTileBits) {
            if (err) *err = "tile view does not cover the qubits";
            return false;
        }
    }
    return true;
}

// Half-tile views (hqml_internal.hpp): the group of full view v on 12 positions.  Low
// positions 0..3 as in the full view; the rotated high qubits split over H1 registers
// (positions 4..7) and H2 registers (8..11); free register positions take other high
// qubits.  Checked: (a) where the statistics of a rotated qubit are taken (H1 for
// positions 0, 1, 4..7; H2 for 8..11) none of its chain neighbours sits at a register
// position of that layout; (b) no qubit at positions 8, 9 neighbours one at 10, 11, and
// none at 4, 5 one at 6, 7 (the diagonal's two per-thread factor tables in H2 or H1).
bool half_view_ok(const int *perm, uint32_t group)
{
    constexpr uint32_t kH1Stat = 0x0F3u, kH1Regs = 0x0F0u, kH2Regs = 0xF00u;
    for (int a = 0; a < kHalfBits; ++a) {
        if (!((group >> a) & 1u)) continue;
        const uint32_t regs = ((kH1Stat >> a) & 1u) ? kH1Regs : kH2Regs;
        for (int b = 0; b < kHalfBits; ++b)
            if (b != a && ((regs >> b) & 1u) && adjacent(perm[a], perm[b])) return false;
    }
    for (int a : {8, 9})
        for (int b : {10, 11})
            if (adjacent(perm[a], perm[b])) return false;
    for (int a : {4, 5})
        for (int b : {6, 7})
            if (adjacent(perm[a], perm[b])) return false;
    return true;
}

bool build_half_view(int n, const ViewDev &full, ViewDevH *out)
{
    std::vector<int> rhigh, fill;
    const uint32_t g = (uint32_t)full.group_mask;
    for (int pos = 4; pos < kTileBits; ++pos)
        if ((g >> pos) & 1u) rhigh.push_back(full.perm[pos]);
    for (int q = kLowQubits; q < n; ++q)
        if (full.inv[q] < 0 || !((g >> full.inv[q]) & 1u)) fill.push_back(q);
    std::sort(fill.rbegin(), fill.rend());   // fillers: highest first
    const int kh = (int)rhigh.size();
    if (kh > 8) return false;
    int perm[kHalfBits];
    uint32_t group = 0;
    for (int nl2 = std::max(0, kh - 4); nl2 <= std::min(4, kh); ++nl2) {
        std::vector<int> pick(kh, 0);
        std::fill(pick.end() - nl2, pick.end(), 1);
        do {
            for (int i = 0; i < kHalfBits; ++i) perm[i] = -1;
            group = g & 3u;
            for (int i = 0; i < kLowQubits; ++i) perm[i] = full.perm[i];
            int p1 = 4, p2 = 8;
            for (int k = 0; k < kh; ++k) {
                const int pos = pick[k] ? p2++ : p1++;
                perm[pos] = rhigh[k];
                group |= 1u << pos;
            }
            std::vector<int> cand = fill;
            bool ok = true;
            for (int pos = 4; pos < kHalfBits && ok; ++pos) {
                if (perm[pos] >= 0) continue;
                ok = false;
                for (size_t ci = 0; ci < cand.size(); ++ci) {
                    perm[pos] = cand[ci];
                    if (half_view_ok(perm, group)) {
                        cand.erase(cand.begin() + (long)ci);
                        ok = true;
                        break;
                    }
                    perm[pos] = -1;
                }
            }
            if (ok && half_view_ok(perm, group)) {
                ViewDevH &d = *out;
                std::memset(&d, 0, sizeof(d));
                int inv[32];
                for (int i = 0; i < 32; ++i) inv[i] = -1;
                for (int i = 0; i < kHalfBits; ++i) {
                    d.perm[i] = perm[i];
                    inv[perm[i]] = i;
                    d.slot_pos[i] = ((group >> i) & 1u) ? full.inv[perm[i]] : kTileBits - 1;
                }
                d.group_mask = (int32_t)group;
                int nt = 0;
                for (int q = 0; q < n; ++q)
                    if (inv[q] < 0) d.tile_q[nt++] = q;
                d.n_tile = nt;
                return nt == n - kHalfBits;
            }
        } while (std::next_permutation(pick.begin(), pick.end()));
    }
    return false;
}

}  // namespace

int stat_tiles(const Plan &p, int compute64)
{
    (void)compute64;   // both compute types run the half-tile adjoint shapes
    return (p.half && !p.small) ? 2 * p.T : p.T;
}

bool make_obs_view(int n, uint32_t xmask, ViewDev *out, std::string *err)
{
    if (n <= kSmallMaxQubits) {
        if (err) *err = "observable views are for the tile path";
        return false;
    }
    ViewDev d;
    std::memset(&d, 0, sizeof(d));
    for (int i = 0; i < 32; ++i) d.inv[i] = -1;
    int pos = 0;
    for (int q = 0; q < kLowQubits; ++q) d.perm[pos++] = q;
    for (int q = kLowQubits; q < n; ++q)   // every high qubit of the X part on chip
        if ((xmask >> q) & 1u) {
            if (pos == kTileBits) {
                if (err) *err = "the X/Y factors of the observable span more than 9 qubits above qubit 3";
                return false;
            }
            d.perm[pos++] = q;
        }
    for (int q = kLowQubits; q < n && pos < kTileBits; ++q)
        if (!((xmask >> q) & 1u)) d.perm[pos++] = q;
    for (int i = 0; i < kTileBits; ++i) d.inv[d.perm[i]] = i;
    int nt = 0;
    for (int q = 0; q < n; ++q)
        if (d.inv[q] < 0) d.tile_q[nt++] = q;
    d.n_tile = nt;
    d.group_mask = 0;
    *out = d;
    return true;
}

// CNOT-chain plan.  The chain maps basis state i to P(i) (bit k = parity of bits 0..k
// of i); it mixes every index bit, so it cannot be applied inside a tile and the
// diagonals of consecutive layers do not merge across it.  Per layer l >= 1 there is
// one pass per view: view 0 reads its input through P^-1 (the previous layer's chain),
// applies diag(r_l) and its group of Ry-layer l; middle views their group; the last
// view its group and diag(p_l).  Pass 0 forms the layer-0 product state and applies
// diag(p_0).  Diagonal table rows: l = diag(p_l), L + l = diag(r_l).  Layer-0
// statistics come from stats-only passes, one per view (pass 0's own backward is one).
static bool make_plan_cnot(Plan &p, int ckpt_block, std::string *err)
{
    const int n = p.n, L = p.L, V = p.V;
    auto slot_of = [&](int v, int q, int sel) { return (sel * 13 + p.views[v].inv[q]) * 3; };
    p.cnot = true;
    p.fwd.push_back(PassPlan{0, true, -1, 0, -1});
    for (int l = 1; l < L; ++l)
        for (int v = 0; v < V; ++v) {
            PassPlan pp{v, false, -1, -1, -1};
            if (v == 0) {
                pp.gather = true;
                pp.diag = L + l;
                pp.rotB = l;
            } else {
                pp.rotA = l;
            }
            if (v == V - 1) pp.diag = l;
            p.fwd.push_back(pp);
        }
    const int P = (int)p.fwd.size();
    for (int v = 1; v < V; ++v) p.stats_only.push_back(v);
    for (int q = 0; q < n; ++q) {
        int v0 = -1;
        for (int v = 0; v < V; ++v) {
            const int pos = p.views[v].inv[q];
            if (pos >= 0 && ((p.views[v].group_mask >> pos) & 1)) v0 = v;
        }
        if (v0 < 0) {
            if (err) *err = "a qubit is rotated by no view";
            return false;
        }
        p.statmap[q] = v0 == 0 ? StatLoc{0, slot_of(0, q, 0)} : StatLoc{P + (v0 - 1), slot_of(v0, q, 0)};
        for (int l = 1; l < L; ++l)
            p.statmap[(size_t)l * n + q] = StatLoc{1 + (l - 1) * V + v0, slot_of(v0, q, v0 == 0 ? 1 : 0)};
    }
    if (ckpt_block > 0) {
        p.c = std::max(1, ckpt_block * V);
        if (p.c >= P) p.c = 0;
    }
    p.nblocks = p.c > 0 ? (P + p.c - 1) / p.c : 1;
    return true;
}

bool make_plan(int n, int L, int ckpt_block, Plan *out, std::string *err, bool cnot)
{
    Plan p;
    p.n = n;
    p.L = L;
    if (n < 1 || n > kMaxQubits) {
        if (err) *err = "n_qubits must be in 1..29";
        return false;
    }
    if (L < 1) {
        if (err) *err = "n_layers must be >= 1";
        return false;
    }
    if (ckpt_block < 0) {
        if (err) *err = "ckpt_block must be >= 0";
        return false;
    }
    p.statmap.assign((size_t)L * n, StatLoc{-1, 0});
    if (n <= kSmallMaxQubits) {
        p.small = true;
        p.V = 1;
        p.T = 1;
        *out = p;
        return true;
    }
    if (!build_views(n, p, err)) return false;
    p.hviews.assign(p.V, ViewDevH{});
    p.half = true;
    for (int v = 0; v < p.V; ++v)
        if (!build_half_view(n, p.views[v], &p.hviews[v])) p.half = false;
    if (!p.half) p.hviews.clear();
    if (cnot) {
        if (!make_plan_cnot(p, ckpt_block, err)) return false;
        *out = p;
        return true;
    }
    const int V = p.V;
    auto group_has = [&](int v, int q) {
        const int pos = p.views[v].inv[q];
        return pos >= 0 && ((p.views[v].group_mask >> pos) & 1);
    };
    auto slot_of = [&](int v, int q, int sel) { return (sel * 13 + p.views[v].inv[q]) * 3; };

    // Pass 0: layer-0 product state, D_0, Ry-layer 1 of view 0's group.
    p.fwd.push_back(PassPlan{0, true, -1, L >= 2 ? 0 : -1, L >= 2 ? 1 : -1});
    int prev = 0;                       // view holding the last slot of the previous layer
    // layer 1's first slot (view 0) is the rotB of pass 0
    std::vector<int> first_view(L, -1), first_pass(L, -1);
    std::vector<std::vector<int>> rotA_pass(L, std::vector<int>(V, -1));
    if (L >= 2) { first_view[1] = 0; first_pass[1] = 0; }
    for (int l = 1; l < L; ++l) {
        std::vector<int> ord;
        ord.push_back(prev);
        for (int k = 1; k < V; ++k) ord.push_back((prev + k) % V);
        for (int k = 1; k + 1 < V; ++k) {           // middle slots: own pass, no diagonal
            rotA_pass[l][ord[k]] = (int)p.fwd.size();
            p.fwd.push_back(PassPlan{ord[k], false, l, -1, -1});
        }
        const int last = ord[V - 1];
        rotA_pass[l][last] = (int)p.fwd.size();
        if (l + 1 < L) {
            first_view[l + 1] = last;
            first_pass[l + 1] = (int)p.fwd.size();
            p.fwd.push_back(PassPlan{last, false, l, l, l + 1});
        } else {
            p.fwd.push_back(PassPlan{last, false, l, -1, -1});
        }
        prev = last;
    }
    const int P = (int)p.fwd.size();
    for (int v = 1; v < V; ++v) p.stats_only.push_back(v);
    // Statistics locations.
    for (int q = 0; q < n; ++q) {
        int v0 = -1;
        for (int v = 0; v < V; ++v)
            if (group_has(v, q)) v0 = v;
        if (v0 < 0) {
            if (err) *err = "a qubit is rotated by no view";
            return false;
        }
        // layer 0
        if (v0 == 0)
            p.statmap[q] = StatLoc{0, slot_of(0, q, 0)};
        else
            p.statmap[q] = StatLoc{P + (v0 - 1), slot_of(v0, q, 0)};
        for (int l = 1; l < L; ++l) {
            if (first_view[l] == v0)
                p.statmap[(size_t)l * n + q] = StatLoc{first_pass[l], slot_of(v0, q, 1)};
            else
                p.statmap[(size_t)l * n + q] = StatLoc{rotA_pass[l][v0], slot_of(v0, q, 0)};
        }
    }
    for (const StatLoc &s : p.statmap)
        if (s.pass < 0) {
            if (err) *err = "statistics map incomplete";
            return false;
        }
    if (ckpt_block > 0) {
        p.c = std::max(1, ckpt_block * (V - 1));
        if (p.c >= P) p.c = 0;           // one block: same as keeping every output
    }
    p.nblocks = p.c > 0 ? (P + p.c - 1) / p.c : 1;
    *out = p;
    return true;
}

Workspace size_workspace(const Plan &p, int max_batch, int storage, int compute64)
{
    Workspace w;
    const size_t B = (size_t)std::max(max_batch, 0);
    const size_t r = compute64 ? 8 : 4;           // bytes of the compute type
    w.state_elems = (size_t)1 << p.n;
    const size_t elem = storage == 1 ? 4 : storage == 2 ? 16 : 8;
    w.state_bytes = B * w.state_elems * elem;
    const size_t Ln = (size_t)p.L * p.n;
    // tables: zyz (6 doubles), frame (1 byte), rot_tf (2 reals), dw (4 reals; 8 with the CNOT plan), H (9
    // doubles), statmap (int2),
    // init_u (4 reals per sample and qubit), views, per-sample E / dL/dE / scratch, loss.
    w.tables_bytes = Ln * (6 * 8 + 1 + 2 * r + 4 * r * (p.cnot ? 2 : 1) + 9 * 8 + 8) + B * p.n * 4 * r +
                     (size_t)(std::max(p.V, 1) + 1) * sizeof(ViewDev) + p.hviews.size() * sizeof(ViewDevH) +
                     B * (8 * 3 + 4) + 64;
    const size_t S_bytes = B * Ln * 3 * 8;
    if (p.small) {
        w.n_saved = 1;
        w.lam_bytes = 0;
        w.state_bytes = B * w.state_elems * 2 * r;   // final state in the compute type (on-chip path)
        w.part_passes = 0;
        w.part_bytes = 0;
        w.total = w.state_bytes + w.tables_bytes + S_bytes + B * r;
        return w;
    }
    const int P = p.n_fwd();
    w.lam_bytes = B * w.state_elems * 2 * r;
    if (p.c == 0) {
        w.n_saved = P;
        w.n_ckpt = 0;
        w.part_passes = p.n_bwd();
    } else {
        w.n_ckpt = p.nblocks - 1;
        w.n_saved = p.c + w.n_ckpt;
        w.part_passes = p.c + (int)p.stats_only.size();
    }
    const int Ts = stat_tiles(p, compute64);
    w.part_bytes = (size_t)w.part_passes * B * Ts * kSlots * r;
    const size_t epart = B * p.T * r;
    if (Ts > kStatChunk) {
        w.tile_chunks = Ts / kStatChunk;
        w.part2_bytes = (size_t)w.part_passes * B * w.tile_chunks * kSlots * 8;
    }
    if (p.T > kTileChunk) w.epart2_bytes = B * (size_t)(p.T / kTileChunk) * 8;
    // the CNOT plan keeps a second lambda buffer (passes that write lambda through the chain)
    w.total = (size_t)w.n_saved * w.state_bytes + w.lam_bytes * (p.cnot ? 2 : 1) + w.part_bytes + w.tables_bytes +
              S_bytes + epart + w.part2_bytes + w.epart2_bytes;
    return w;
}

int gbg_blocks_per_sample(int n)
{
    const size_t half = (size_t)1 << (n - 1);
    return (int)((half + kGbgPairsPerBlock - 1) / kGbgPairsPerBlock);
}

Workspace size_workspace_gbg(int n, int L, int max_batch)
{
    Workspace w;
    const size_t B = (size_t)max_batch;
    const size_t nblk = (size_t)gbg_blocks_per_sample(n);
    const size_t n_params = (size_t)L * n * 3;
    w.state_elems = (size_t)1 << n;
    w.state_bytes = B * w.state_elems * 8;
    w.n_saved = 1;
    w.lam_bytes = w.state_bytes;
    w.part_passes = 0;
    w.part_bytes = n_params * B * nblk * 8;
    w.tile_chunks = nblk > (size_t)kTileChunk ? (int)(nblk / kTileChunk) : 0;
    w.epart2_bytes = B * (size_t)w.tile_chunks * 8;
    // theta copy, dL/dE, E scratch, loss, per-block <O> partials
    w.tables_bytes = n_params * 4 + B * 16 + 64 + B * nblk * 4;
    w.total = w.state_bytes + w.lam_bytes + w.part_bytes + w.epart2_bytes + w.tables_bytes;
    return w;
}

std::string describe_plan(const Plan &p)
{
    std::string s = "{";
    char buf[256];
    std::snprintf(buf, sizeof buf,
                  "\"n\":%d,\"L\":%d,\"small\":%s,\"cnot\":%s,\"V\":%d,\"T\":%d,\"c\":%d,\"nblocks\":%d,", p.n, p.L,
                  p.small ? "true" : "false", p.cnot ? "true" : "false", p.V, p.T, p.c, p.nblocks);
    s += buf;
    s += "\"views\":[";
    for (size_t v = 0; v < p.views.size(); ++v) {
        const ViewDev &d = p.views[v];
        s += v ? ",{" : "{";
        s += "\"perm\":[";
        for (int i = 0; i < kTileBits; ++i) {
            std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", d.perm[i]);
            s += buf;
        }
        s += "],\"tile_q\":[";
        for (int i = 0; i < d.n_tile; ++i) {
            std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", d.tile_q[i]);
            s += buf;
        }
        std::snprintf(buf, sizeof buf, "],\"group_mask\":%d}", d.group_mask);
        s += buf;
    }
    s += "],\"half\":";
    s += p.half ? "true" : "false";
    s += ",\"hviews\":[";
    for (size_t v = 0; v < p.hviews.size(); ++v) {
        const ViewDevH &d = p.hviews[v];
        s += v ? ",{" : "{";
        s += "\"perm\":[";
        for (int i = 0; i < kHalfBits; ++i) {
            std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", d.perm[i]);
            s += buf;
        }
        s += "],\"slot_pos\":[";
        for (int i = 0; i < kHalfBits; ++i) {
            std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", d.slot_pos[i]);
            s += buf;
        }
        s += "],\"tile_q\":[";
        for (int i = 0; i < d.n_tile; ++i) {
            std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", d.tile_q[i]);
            s += buf;
        }
        std::snprintf(buf, sizeof buf, "],\"group_mask\":%d}", d.group_mask);
        s += buf;
    }
    s += "],\"passes\":[";
    for (size_t i = 0; i < p.fwd.size(); ++i) {
        const PassPlan &q = p.fwd[i];
        std::snprintf(buf, sizeof buf,
                      "%s{\"view\":%d,\"init\":%s,\"rotA\":%d,\"diag\":%d,\"rotB\":%d,\"gather\":%s}", i ? "," : "",
                      q.view, q.init ? "true" : "false", q.rotA, q.diag, q.rotB, q.gather ? "true" : "false");
        s += buf;
    }
    s += "],\"stats_only\":[";
    for (size_t i = 0; i < p.stats_only.size(); ++i) {
        std::snprintf(buf, sizeof buf, "%s%d", i ? "," : "", p.stats_only[i]);
        s += buf;
    }
    s += "],\"statmap\":[";
    for (size_t i = 0; i < p.statmap.size(); ++i) {
        std::snprintf(buf, sizeof buf, "%s[%d,%d]", i ? "," : "", p.statmap[i].pass, p.statmap[i].slot);
        s += buf;
    }
    s += "]}";
    return s;
}

}  // namespace hqml
