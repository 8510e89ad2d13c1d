// Device hooks for the host-only build of the encoder, model, blob and planning code
// (the sanitizer build): with no HIP unit linked in, no blob ever holds device memory,
// so releasing a blob's device copy has nothing to do.
#include "ep_internal.h"

void ep_device_release(ep::Blob*) {}
