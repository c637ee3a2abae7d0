// Attention forward with a dense mask ("SAFE-DiT" Eq. 2 with m given): the instances
// that read a Boolean or additive mask tile alongside each key tile.  This is the call
// that the Eq. 8 rewrite removes for masks in R; it stays for masks outside R and
// measures what the rewrite saves.  No key-length form: a padding mask is either
// given as a mask here or as per-sample lengths to the mask-free instances.
#include "attn_kernel.h"

namespace safe {
namespace {

template <int D, int MT>
hipError_t dispatch_gather(const AttnParams& p, bool gather, hipStream_t s) {
  return gather ? launch<D, true, false, MT, 1>(p, s) : launch<D, false, false, MT, 1>(p, s);
}

template <int D>
hipError_t dispatch_mt(const AttnParams& p, bool gather, int mt, hipStream_t s) {
  switch (mt) {
    case kMaskBool: return dispatch_gather<D, kMaskBool>(p, gather, s);
    case kMaskBf16: return dispatch_gather<D, kMaskBf16>(p, gather, s);
    case kMaskF16: return dispatch_gather<D, kMaskF16>(p, gather, s);
    case kMaskF32: return dispatch_gather<D, kMaskF32>(p, gather, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int MT>
int resident_gather(bool gather) {
  return gather ? resident_workgroups<D, true, false, MT, 1>() : resident_workgroups<D, false, false, MT, 1>();
}

template <int D>
int resident_mt(bool gather, int mt) {
  switch (mt) {
    case kMaskBool: return resident_gather<D, kMaskBool>(gather);
    case kMaskBf16: return resident_gather<D, kMaskBf16>(gather);
    case kMaskF16: return resident_gather<D, kMaskF16>(gather);
    case kMaskF32: return resident_gather<D, kMaskF32>(gather);
    default: return 0;
  }
}

}  // namespace

hipError_t attn_masked_dispatch(const AttnParams& p, int d, bool gather, int mt, hipStream_t s) {
  switch (d) {
    case 32: return dispatch_mt<32>(p, gather, mt, s);
    case 64: return dispatch_mt<64>(p, gather, mt, s);
    case 72: return dispatch_mt<72>(p, gather, mt, s);
    case 96: return dispatch_mt<96>(p, gather, mt, s);
    case 128: return dispatch_mt<128>(p, gather, mt, s);
    default: return hipErrorInvalidValue;
  }
}

int attn_masked_resident(int d, bool gather, int mt) {
  switch (d) {
    case 32: return resident_mt<32>(gather, mt);
    case 64: return resident_mt<64>(gather, mt);
    case 72: return resident_mt<72>(gather, mt);
    case 96: return resident_mt<96>(gather, mt);
    case 128: return resident_mt<128>(gather, mt);
    default: return 0;
  }
}

}  // namespace safe
