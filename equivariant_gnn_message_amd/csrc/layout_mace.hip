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
const FwdLauncher kF32[] = {launch_fwd_pipe<L, float, 4, 2>, launch_fwd<L, float, 2, 1>,
                            launch_fwd_pipe<L, float, 2, 1>, launch_fwd_pipe<L, float, 4, 1>};
const FwdLauncher kBF16[] = {launch_fwd_pipe<L, bf16_bits, 4, 2>, launch_fwd<L, bf16_bits, 2, 1>,
                             launch_fwd_pipe<L, bf16_bits, 2, 1>};
const BwdLauncher kBwd[] = {launch_bwd_pipe<L, 2, 1>, launch_bwd<L, 4, 2>, launch_bwd<L, 2, 1>,
                            launch_bwd_pipe<L, 4, 2>};

const FwdLauncher kSenderF32[] = {launch_fwd_pipe<LS, float, 4, 2>};
const FwdLauncher kSenderBF16[] = {launch_fwd_pipe<LS, bf16_bits, 4, 2>};
const BwdLauncher kSenderBwd[] = {launch_bwd_pipe<LS, 2, 1>};

#define E3C_N(a) (int)(sizeof(a) / sizeof((a)[0]))

}  // namespace

const KernelSet* kernels_mace() {
  static const KernelSet k = {
    L::C, L::XCODE, L::L, L::OCODE, &kTables, kCG.v,
    {kF32, E3C_N(kF32), kBF16, E3C_N(kBF16), kBwd, E3C_N(kBwd), launch_bwd_pipe<L, 2, 1, true>,
     launch_jvp_pipe<L, float, 2, 1, false>, launch_jvp_pipe<L, bf16_bits, 2, 1, true>},
    {kSenderF32, 1, kSenderBF16, 1, kSenderBwd, 1, launch_bwd_pipe<LS, 2, 1, true>,
     launch_jvp_pipe<LS, float, 2, 1, false>, launch_jvp_pipe<LS, bf16_bits, 2, 1, true>},
  };
  return &k;
}

}  // namespace e3c
