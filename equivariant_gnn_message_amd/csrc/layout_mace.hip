// Kernels of the layout 128x0e+128x1o, lmax 3 -> 128x(0e+1o+2e+3o).
#include "conv_kernels.h"

namespace e3c {
namespace {

using L = Layout<128, natural_code(1), 3, natural_code(3)>;
using LS = SenderOrdered<L>;

constexpr LayoutTables kTables = L::T;
constexpr CGValues<L::NNZ> kCG = L::CG;

// Variant 0 of each list is the default (the fastest measured on MI355X for
// the workload of this layout); the others stay selectable for comparison.
// Defaults run one wave per work-group: a work-group's slot is released only
// when its last wave ends, so single-wave work-groups free each wave's slot
// as soon as it is done (measured on MI355X, training step on the MACE-scale
// graph: forward 0.660 against 0.667 ms, reverse 1.364 against 1.369 ms with
// four-wave work-groups, forward variant 4 and reverse variant 7).  The
// reverse default reads the two groups' y rows and sender indices through
// the scalar cache: 1.347 against 1.366 ms (reverse variant 8).
const FwdLauncher kF32[] = {launch_fwd_pipe<L, float, 4, 2, false, false, false, 1>, launch_fwd<L, float, 2, 1>,
                            launch_fwd_pipe<L, float, 2, 1>, launch_fwd_pipe<L, float, 4, 1>,
                            launch_fwd_pipe<L, float, 4, 2>};
const FwdLauncher kBF16[] = {launch_fwd_pipe<L, bf16_bits, 4, 2>, launch_fwd<L, bf16_bits, 2, 1>,
                             launch_fwd_pipe<L, bf16_bits, 2, 1>};
const BwdLauncher kBwd[] = {launch_bwd_tile<L, 4, 16, false, 1, true, true>, launch_bwd_pipe<L, 2, 1>,
                            launch_bwd<L, 4, 2>, launch_bwd<L, 2, 1>, launch_bwd_pipe<L, 4, 2>,
                            launch_bwd_tile<L, 4, 8, false, 1, true, true>,
                            launch_bwd_tile<L, 4, 32, false, 1, true, true>, launch_bwd_tile<L, 4, 16>,
                            launch_bwd_tile<L, 4, 16, false, 1>};

const FwdLauncher kSenderF32[] = {launch_fwd_pipe<LS, float, 4, 2, false, false, false, 1>};
const FwdLauncher kSenderBF16[] = {launch_fwd_pipe<LS, bf16_bits, 4, 2>};
const BwdLauncher kSenderBwd[] = {launch_bwd_pipe<LS, 2, 1, false, 1>};

#define E3C_N(a) (int)(sizeof(a) / sizeof((a)[0]))

}  // namespace

const KernelSet* kernels_mace() {
  static const KernelSet k = {
    L::C, L::XCODE, L::L, L::OCODE, &kTables, kCG.v,
    {kF32, E3C_N(kF32), kBF16, E3C_N(kBF16), kBwd, E3C_N(kBwd), launch_bwd_pipe<L, 2, 1, true, 1>,
     launch_jvp_pipe<L, float, 2, 1, false, 1>, launch_jvp_pipe<L, bf16_bits, 2, 1, true, 1>, nullptr,
     launch_bwd_pairs<L, 2, 16, 1>, nullptr, nullptr, launch_fwd_pipe<L, float, 2, 1, false, false, true, 1>},
    {kSenderF32, 1, kSenderBF16, 1, kSenderBwd, 1, launch_bwd_pipe<LS, 2, 1, true>,
     launch_jvp_pipe<LS, float, 2, 1, false>, launch_jvp_pipe<LS, bf16_bits, 2, 1, true>},
  };
  return &k;
}

}  // namespace e3c
