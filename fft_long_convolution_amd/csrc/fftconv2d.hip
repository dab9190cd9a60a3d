// fftconv2d.hip -- placeholder translation unit for the 2D path.
#include "kernels.h"
