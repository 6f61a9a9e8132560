// One kernel class of the fused CGTP convolution (the class is chosen at build time
// with -DCGTP_CONV_CLASS=<k>; the build compiles this file once per class).
#include "conv_kernel.hpp"

#ifndef CGTP_CONV_CLASS
#error "CGTP_CONV_CLASS must be defined"
#endif

namespace cgtp {
template hipError_t launch_conv_class<CGTP_CONV_CLASS, float>(const ConvArgsT<float>& args, hipStream_t s,
                                                              hipEvent_t ev_start, hipEvent_t ev_stop);
#if CGTP_CONV_CLASS < 7   // the classes with variants of l <= kBwdLmax
template hipError_t launch_conv_bwd_class<CGTP_CONV_CLASS>(const ConvArgsT<float>& args, hipStream_t s);
#endif
#if CGTP_CONV_CLASS < 7   // kNumClassesF64
static_assert(CGTP_CONV_CLASS < kNumClassesF64, "fp64 class range");
template hipError_t launch_conv_class<CGTP_CONV_CLASS, double>(const ConvArgsT<double>& args, hipStream_t s,
                                                               hipEvent_t ev_start, hipEvent_t ev_stop);
#endif
}  // namespace cgtp
