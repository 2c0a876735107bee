// Prefill-chunk indexer kernels (added with the prefill entry points).
#include "ls_device.h"
#include "ls_launch.h"
