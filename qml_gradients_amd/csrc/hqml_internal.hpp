// Internal structures shared by the host scheduler (hqml_plan.cpp, hqml_abi.cpp)
// and the gfx950 kernels (hqml_kernels.hip).  Not part of the public ABI.
//
// Method: Kawase, "Fast and memory-efficient classical simulation of quantum
// machine learning via forward and backward gate fusion" (arXiv:2603.02804),
// hugo-pages summary sections 1.2-1.4: forward gate fusion applies a block of
// gates to a state kept on chip and writes the block output once; backward gate
// fusion re-derives each earlier state on chip with U^dagger while forming the
// adjoint gradient terms and propagating lambda.
//
// Layer algebra used by the kernels.  Layer l applies U_{l,q} = Rz(g) Ry(b) Rx(a)
// to every qubit q (R_s(t) = exp(-i t s/2)) and then the CZ chain.  U is in SU(2),
// so it factors exactly as
//     U_{l,q} = diag(p, conj p) * Ry(beta) * diag(r, conj r),  beta in [0, pi],
// (cos(beta/2) = |U00|, sin(beta/2) = |U10|, p r = U00/|U00|, conj(p) r = U10/|U10|).
// Between the real rotation layers Ry(beta_l) and Ry(beta_{l+1}) every factor is
// diagonal: left factors of layer l, the CZ chain of layer l, right factors of
// layer l+1.  They merge into one diagonal
//     D_l(i) = czsign_l(i) * prod_q (bit_q(i) ? conj(w_{l,q}) : w_{l,q}),
//     w_{l,q} = p_{l,q} r_{l+1,q},
// so the simulated circuit is
//     psi_0 (product state, all of layer 0's right factors and Ry applied),
//     D_0, Ry-layer 1, D_1, ..., Ry-layer L-1,
// and the trailing diagonal (layer L-1's left factors and CZ chain) is dropped:
// it commutes with the (diagonal) observable and does not change E or any gradient.  Gradients are taken
// at the point P_l just after Ry-layer l: with S_s = Im<mu|s_q|psi> (s = X, Y, Z
// on qubit q, mu the back-propagated O psi_M),
//     dE/dtheta[l][q][a] = sum_s H[l][q][a][s] * S_s,
// where H holds the Pauli coefficients of p-conjugated rotated generators
// (computed in k_prep_tables).  A Pauli frame (k_prep_frame) then keeps every
// simulated rotation in the form f [[1, -k], [k, 1]] with |k| <= 1.
#pragma once
#include <stdint.h>

namespace hqml {

// ---- tile geometry (n > kTileBits) ----
// A tile holds 2^13 amplitudes of one sample: 13 "local positions", each bound to
// one global qubit by the tile's view.  256 threads x 32 registers.
// Layout L1 (global-memory layout):  regs  <- positions 4..8
//                                     lanes <- positions 0,1,2,3,9,10
//                                     waves <- positions 11,12
// Layout L2 (after one LDS transpose): regs  <- positions 0,1,9,10,11
//                                     lanes <- positions 2..7
//                                     waves <- positions 8,12
// Rotations act on register bits only, so a view rotates qubits at positions
// {4..8} (in L1) and {0,1,9,10,11} (in L2).  Positions 0..3 always hold global
// qubits 0..3 (any order), so 16 consecutive amplitudes (128 bytes) are
// contiguous in memory for every view.
constexpr int kTileBits = 13;
constexpr int kRegBits = 5;
constexpr int kRegs = 32;
constexpr int kThreads = 256;
constexpr int kGbgPairsPerBlock = 4096; // gate-by-gate kernels: amplitude pairs per workgroup
constexpr int kTileChunk = 256;     // tiles per first-stage <O> reduction block (samples with more tiles)
constexpr int kStatChunk = 64;      // tiles per first-stage statistics reduction block (samples with more
                                    // tiles): a block reads whole rows of partials, coalesced
constexpr int kSlots = 80;           // per-tile statistics slots: (sel*13 + pos)*3 + pauli
constexpr int kMaxQubits = 29;
constexpr int kSmallMaxQubits = 13;  // whole state of one sample in one workgroup
constexpr uint32_t kRotatableMask = 0x0FF3u;  // positions 0,1,4..11

struct ViewDev {
    int32_t perm[kTileBits];   // global qubit held at local position
    int32_t inv[32];           // local position of a global qubit, -1 if it is a tile bit
    int32_t n_tile;            // number of tile-index bits
    int32_t tile_q[32];        // global qubit of tile-index bit k
    int32_t group_mask;        // local positions whose qubits this view rotates
    int32_t pad[3];
};

// Half tile of the adjoint pass (hqml_kernels.hip, k_tile_bwdh): 2^12 amplitudes, 256
// threads x 16 registers, so that four workgroups share a compute unit (two in fp64).
// Layout H1 (global-memory layout): regs  <- positions 4..7
//                                    lanes <- positions 0,1,2,3,8,9
//                                    waves <- positions 10,11
// Layout H2 (after one LDS transpose): regs  <- positions 8..11
//                                    lanes <- positions 0..5
//                                    waves <- positions 6,7
// Positions 0 and 1 are lane bits 0 and 1 in both layouts; their rotations and
// statistics take the partner lane's amplitude through a DPP quad permutation.  A half
// view rotates the same group of qubits as the full view of the same index: its rotated
// low qubits at 0, 1, the other low qubits at 2, 3, its rotated high qubits at 4..11.
constexpr int kHalfBits = 12;
constexpr int kHalfRegs = 16;

struct ViewDevH {
    int32_t perm[kHalfBits];       // global qubit held at local position
    int32_t slot_pos[kHalfBits];   // statistics slot position of that qubit: its position in the
                                   // full view (so the statistics land where the full-tile kernel
                                   // puts them); 12 (a slot nobody reads) where it is not rotated
    int32_t n_tile;                // number of tile-index bits (n - 12)
    int32_t tile_q[32];            // global qubit of tile-index bit k
    int32_t group_mask;            // local positions whose qubits this view rotates
    int32_t pad[2];
};

enum PassFlags : int {
    PF_INIT = 1,         // generate the layer-0 product state instead of loading a state
    PF_EMIT_E = 2,       // write per-tile <O> partial sums
    PF_STORE = 4,        // forward: write the pass output
    PF_FUSED = 8,        // forward ops of the (last) pass followed by its backward ops
    PF_STATS_ONLY = 16,  // backward: layer-0 statistics of this view only (no state update)
    PF_SEED = 32,        // backward: lambda = O psi formed from the pass output (last pass)
    PF_CNOT = 64,        // CNOT-chain plan: diagonals are plain single-qubit factors (no CZ
                         // signs); backward shapes of that plan
    PF_GATHER = 128,     // forward: read the input at P^-1(i) (the CNOT chain);
                         // backward: write lambda back to P^-1(i)
    PF_OBS_NEG = 256,    // observable pass: the Pauli string carries an extra sign -1
    PF_HALF = 512        // backward: the general shape on half tiles (k_tile_bwdh)
};

struct TilePassArgs {
    const void *psi_in;     // fwd: input state (previous pass output); bwd: saved output of this pass
    void *psi_out;          // fwd: output state
    // Arrays below hold the compute type R of the kernel (float or double).
    void *lam;              // bwd: adjoint state, complex R, updated in place
    void *e_part;           // [B][T] per-tile <O> partial sums
    void *stat_part;        // [B][T * stat_mul][kSlots] per-tile gradient statistics of this pass
    const void *rot_tf;     // [L][n][2]: tan form (k, f) of the real rotation
    const void *dw;         // [L][n][4]: factors (f0, f1) of qubit q in D_l
    const void *init_u;     // [B][n][4]: (u0.re, u0.im, u1.re, u1.im) layer-0 product factors
    const ViewDev *view;
    const ViewDevH *hview;  // bwd with PF_HALF: the half view of the same group
    int n;
    int L;
    int T;                  // tiles per sample = 2^(n-13)
    int rotA;               // first rotation layer of the pass (-1: none)
    int diag;               // diagonal layer D_l (-1: none)
    int rotB;               // second rotation layer (-1: none)
    int flags;
    int sample0;            // first sample of this launch (the grid covers samples sample0 ..)
    int stat_mul;           // bwd: statistics partials per tile (2 when the context's adjoint
                            // runs on half tiles: full-tile passes write theirs and a zero row)
    uint32_t obs;           // observable: Z part of the Pauli string (qubit mask)
    uint32_t obs_x;         // observable: X part (qubits in both masks carry Y = iXZ)
};

struct SmallArgs {
    // Arrays hold the compute type R of the kernel (float or double).
    const void *init_u;     // [B][n][4]
    const void *rot_tf;     // [L][n][2]
    const void *dw;         // [L][n][4]
    void *psi_save;         // [B][2^n][2]: final state (forward mode writes, backward mode reads)
    void *e_out;            // [B] per-sample <O> (R, from an fp64 in-block sum)
    double *stats;          // [B][L][n][3] per-sample statistics S_s at point P_l
    int n;
    int L;
    int mode;               // 0: forward only; 1: backward only (from psi_save); 2: both
    int ent;                // entangler closing each layer: 0 CZ chain, 1 CNOT chain
    uint32_t obs;           // observable: Z part of the Pauli string (qubit mask)
    uint32_t obs_x;         // observable: X part (qubits in both masks carry Y = iXZ)
};

}  // namespace hqml
